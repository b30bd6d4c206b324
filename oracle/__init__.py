"""fp64 CPU oracle for causal / sliding-window grouped-query attention.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may
import it. It shares no code with the HIP path and imports nothing from the product package.
"""
from .attention import (  # noqa: F401
    cols_dkdv, backward, document_of, forward, forward_backward, head_rows, kv_head, probabilities,
    rows_dq, rows_forward, visible_mask,
)
from .compare import rel_l2  # noqa: F401
from .paged import gather_sequence, paged_forward  # noqa: F401
