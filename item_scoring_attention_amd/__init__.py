"""Multiple-item scoring (MIS) hot path for AMD Instinct MI355X (gfx950).

The computation lives in ``libmis.so`` (HIP kernels behind the C ABI of
``include/mis.h``); this package is its ctypes binding. The calls:

* ``mis_build_segments``: per-token item/position ids, readout positions and
  per-tile classes from prefix lengths and item offsets;
* ``mis_apply_rope``: rotary embedding of Q and K at the reused positions;
* ``mis_attention_prefill``: MIS prefill attention on bf16 MFMA (or fp32);
  ``mis_attention_append``: the same for item rows only, against a cached prefix;
  ``mis_attention_prefill_rope`` / ``mis_attention_append_rope``: the same with
  Q rotated inside the kernel from a ``mis_rope_table`` (K rotated beforehand
  by ``mis_apply_rope`` with ``q=None``);
* ``mis_score_labels``: readout gather, LM-head contraction and full-vocab
  logsumexp, writing one label-score row per item (``mis_score_labels_at``:
  at any token rows, e.g. several readout markers per item;
  ``mis_score_labels_noalloc``: with the library's own per-GPU scratch, for
  callers that cannot allocate).

``pack_requests`` (host only) turns queries, candidate items and a delimiter
token into the packed token ids and the offsets ``mis_build_segments`` takes.
"""
from ._lib import (  # noqa: F401
    LIB_PATH,
    MIS_BF16,
    MIS_ERR_ARG,
    MIS_ERR_HIP,
    MIS_ERR_LABEL,
    MIS_ERR_SEGMENTS,
    MIS_ERR_UNSUPPORTED,
    MIS_ERR_WORKSPACE,
    MIS_F32,
    MIS_MAX_LABELS,
    MIS_SCORE_SCRATCH_BYTES,
    MIS_OK,
    MisError,
    MisSegments,
    MisValueError,
    SIGNATURES,
    Segments,
    attention_kernel_name,
    last_error,
    load,
    mis_apply_rope,
    mis_attention_append,
    mis_attention_append_rope,
    mis_attention_prefill,
    mis_attention_prefill_rope,
    mis_attention_tile_shape,
    mis_build_segments,
    mis_rope_table,
    mis_rope_table_bytes,
    mis_score_labels,
    mis_score_labels_at,
    mis_score_labels_noalloc,
    mis_score_workspace_bytes,
    mis_segments_bytes,
    score_kernel_name,
    set_kernel_choice,
    version,
)
from .pack import Packed, build_packed_segments, pack_requests  # noqa: F401,E402
