"""fp64 CPU oracle for multiple-item scoring: test infrastructure, never the product path.

Only the test suite, the smoke check and the benchmark's CPU-baseline leg
import this package. See ``oracle.mis`` for what it computes and the
passages of the pages each function follows.
"""
from .mis import (  # noqa: F401
    as_f64,
    attention,
    build_segments,
    causal_attention,
    label_scores,
    logits,
    mask_rows,
    mis_mask,
    rope,
    sis_attention,
    sis_rope_attention,
    sis_scores,
    tile_classes,
    visible_pairs,
)
