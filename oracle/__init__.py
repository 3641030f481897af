"""CPU oracle for exact attention -- TEST INFRASTRUCTURE, not part of the product.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import this package.  The GPU library never calls it and shares no code with it.
See ``oracle/attention.py`` for what each function computes and which passage
of the pages it follows.
"""

from .attention import (  # noqa: F401
    visible_mask,
    block_visible,
    distance_bias,
    scores,
    attention_forward,
    attention_forward_rows,
    attention_probabilities,
    attention_backward,
    tiled_online_forward,
    row_block_summary,
    tile_classes,
)
