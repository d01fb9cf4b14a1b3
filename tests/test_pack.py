"""The token-level packer (host code): queries, candidate items and a
delimiter token into one packed MIS batch (From Generation to Scoring §4.1,
Eq. 3; SGLang blog, "Multi-item-scoring": every item closed by the
delimiter, whose logits are read)."""
import numpy as np
import pytest

import oracle
from item_scoring_attention_amd import pack_requests


def test_hand_worked_example():
    p = pack_requests([([5, 6, 7], [[1, 2], [3], []])], delimiter_id=9)
    assert p.token_ids.tolist() == [5, 6, 7, 1, 2, 9, 3, 9, 9]
    assert p.cu_seqlens.tolist() == [0, 9]
    assert p.prefix_lens.tolist() == [3]
    assert p.cu_items.tolist() == [0, 3]
    assert p.item_starts.tolist() == [3, 6, 8]
    # each item is read at its closing delimiter (the oracle's readout rule)
    seg = oracle.build_segments(p.cu_seqlens, p.prefix_lens, p.cu_items, p.item_starts)
    assert seg["readout_pos"].tolist() == [5, 7, 8]
    for a in (p.token_ids, p.cu_seqlens, p.prefix_lens, p.cu_items, p.item_starts):
        assert a.dtype == np.int32


def test_requests_pack_one_after_another():
    p = pack_requests([([1], [[2, 3]]), ([4, 5], []), ([6], [[7], [8, 8, 8]])], delimiter_id=0)
    assert p.token_ids.tolist() == [1, 2, 3, 0, 4, 5, 6, 7, 0, 8, 8, 8, 0]
    assert p.cu_seqlens.tolist() == [0, 4, 6, 13]
    assert p.prefix_lens.tolist() == [1, 2, 1]
    assert p.cu_items.tolist() == [0, 1, 1, 3]
    assert p.item_starts.tolist() == [1, 1, 3]        # request-relative
    seg = oracle.build_segments(p.cu_seqlens, p.prefix_lens, p.cu_items, p.item_starts)
    assert seg["readout_pos"].tolist() == [3, 8, 12]  # packed
    assert p.num_requests == 3 and p.total_items == 3


def test_offsets_agree_with_the_oracle_segments():
    rng = np.random.default_rng(7)
    reqs = []
    for _ in range(5):
        q = rng.integers(0, 1000, size=int(rng.integers(0, 40)))
        items = [rng.integers(0, 1000, size=int(rng.integers(0, 12))) for _ in range(int(rng.integers(0, 9)))]
        reqs.append((q, items))
    p = pack_requests(reqs, delimiter_id=1001)
    seg = oracle.build_segments(p.cu_seqlens, p.prefix_lens, p.cu_items, p.item_starts)
    assert (p.token_ids[seg["readout_pos"]] == 1001).all()
    # every item's tokens, then its delimiter, sit at its segment in order
    n = 0
    for r, (q, items) in enumerate(reqs):
        base = int(p.cu_seqlens[r])
        assert np.array_equal(p.token_ids[base:base + len(q)], q)
        assert (seg["item_id"][base:base + len(q)] == -1).all()
        for c in items:
            rows = np.nonzero(seg["item_id"] == n)[0]
            assert np.array_equal(p.token_ids[rows], np.append(c, 1001))
            # reused positions: the item continues right after the query
            assert np.array_equal(seg["pos_id"][rows], len(q) + np.arange(len(c) + 1))
            n += 1


@pytest.mark.parametrize("reqs, delim", [
    ([([1, -2], [])], 0),          # negative id
    ([([1.5], [])], 0),            # not an integer
    ([([1], [[2]], "x")], 0),      # not a (query, items) pair
    ([([1], [[[2]]])], 0),         # an item that is not flat
    ([([1], [])], -1),             # bad delimiter
    ([([], [])], 0),               # an empty request
])
def test_malformed_input_raises(reqs, delim):
    with pytest.raises(ValueError):
        pack_requests(reqs, delimiter_id=delim)


def test_empty_batch():
    p = pack_requests([], delimiter_id=3)
    assert p.token_ids.size == 0 and p.cu_seqlens.tolist() == [0] and p.total_items == 0
