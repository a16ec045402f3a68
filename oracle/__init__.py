"""fp64 CPU oracle for exact attention (test infrastructure; never part of the product path)."""
from .attention import (  # noqa: F401
    backward,
    backward_head,
    forward,
    forward_head,
    forward_head_rows,
    masked_scores,
    online_softmax_forward_head,
    row_softmax,
    scalar_forward_head,
)
