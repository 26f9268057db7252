"""CPU oracle for Sliding Tile Attention (test infrastructure only).

This package is the checker, not the product: only the tests, the smoke
check and the benchmark's CPU-baseline leg may import it. The HIP library
never calls it and shares no code with it.
"""

from .sta_oracle import (  # noqa: F401
    TILE,
    TEXT_SLOTS,
    window_start,
    allowed_mask,
    key_tiles_of_query_tile,
    query_rows_seeing,
    sta_reference,
    sta_reference_backward,
)
from .hilbert_oracle import (  # noqa: F401
    hilbert_d2xy,
    hilbert_xy2d,
    hilbert_token_order,
    hilbert_allowed_mask,
    hilbert_reference,
    block_counts,
)
