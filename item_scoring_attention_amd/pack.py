"""Token-level packer: the scoring problem as the pages state it (a query,
candidate items and a delimiter token) as one packed MIS prefill.

From Generation to Scoring, §4.1 (Eq. 3): the items follow the shared query
prefix in one sequence and are scored by a single prefill. SGLang blog
("Multi-item-scoring"): every item is closed by the delimiter token, and the
next-token logits at that delimiter give the item's label scores. Several
requests pack one after another (variable-length batch, no attention across
requests).

The offsets ``pack_requests`` returns are exactly the host metadata that
``mis_build_segments`` takes; the per-token ids and each item's readout
position (its closing delimiter) come from the builder. Pure host code: no
GPU work happens here.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Sequence, Tuple

import numpy as np


@dataclass
class Packed:
    """One packed MIS batch.

    token_ids   [T]   int32: per request, the query tokens, then each item's
                      tokens followed by the delimiter;
    cu_seqlens  [B+1] int32: packed offset of each request;
    prefix_lens [B]   int32: query length of each request;
    cu_items    [B+1] int32: global index of each request's first item;
    item_starts [N]   int32: request-relative start of each item.
    """

    token_ids: np.ndarray
    cu_seqlens: np.ndarray
    prefix_lens: np.ndarray
    cu_items: np.ndarray
    item_starts: np.ndarray

    @property
    def num_requests(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_items(self) -> int:
        return int(self.item_starts.shape[0])


def _ids(x, what: str) -> np.ndarray:
    a = np.asarray(x)
    if a.ndim != 1:
        raise ValueError(f"{what} must be a 1-D sequence of token ids")
    if a.size and not np.issubdtype(a.dtype, np.integer):
        raise ValueError(f"{what} must hold integer token ids")
    if a.size and (a.min() < 0 or a.max() > np.iinfo(np.int32).max):
        raise ValueError(f"{what} holds a token id outside [0, 2^31)")
    return a.astype(np.int32)


def pack_requests(requests: Sequence[Tuple[Sequence[int], Sequence[Sequence[int]]]], delimiter_id: int) -> Packed:
    """Pack ``[(query_ids, [item_ids, ...]), ...]`` into one batch.

    Request r becomes ``query_r, item_r0, d, item_r1, d, ...`` with ``d`` the
    delimiter; an item may be empty (then it is the delimiter alone). A
    request without items is a plain causal prefill of its query. Raises
    ValueError for malformed input (non-integer or negative ids, an empty
    request, a batch longer than 2^31 - 1 tokens).
    """
    if not (0 <= int(delimiter_id) <= np.iinfo(np.int32).max):
        raise ValueError("delimiter_id must be a token id in [0, 2^31)")
    d = np.array([delimiter_id], dtype=np.int32)
    pieces, cu_seqlens, prefix_lens, cu_items, item_starts = [], [0], [], [0], []
    total = 0
    for r, req in enumerate(requests):
        try:
            query, items = req
        except (TypeError, ValueError):
            raise ValueError(f"request {r} must be a (query_ids, items) pair") from None
        q = _ids(query, f"request {r} query")
        pieces.append(q)
        length = q.size
        prefix_lens.append(q.size)
        for i, item in enumerate(items):
            c = _ids(item, f"request {r} item {i}")
            item_starts.append(length)
            pieces += [c, d]
            length += c.size + 1
        if length == 0:
            raise ValueError(f"request {r} has no query tokens and no items")
        total += length
        if total > np.iinfo(np.int32).max:
            raise ValueError("packed batch longer than 2^31 - 1 tokens")
        cu_seqlens.append(total)
        cu_items.append(len(item_starts))
    i32 = lambda x: np.asarray(x, dtype=np.int32)
    tokens = np.concatenate(pieces) if pieces else np.zeros(0, dtype=np.int32)
    return Packed(tokens.astype(np.int32), i32(cu_seqlens), i32(prefix_lens), i32(cu_items), i32(item_starts))


def build_packed_segments(packed: Packed, block_m: int, block_n: int, dev_buf=None, stream=None):
    """``mis_build_segments`` on a packed batch's offsets."""
    from ._lib import mis_build_segments
    return mis_build_segments(packed.cu_seqlens, packed.prefix_lens, packed.cu_items, packed.item_starts,
                              block_m, block_n, dev_buf=dev_buf, stream=stream)
