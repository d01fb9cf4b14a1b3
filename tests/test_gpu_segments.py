"""GPU segment builder vs the oracle: bit-exact item ids, positions, readouts, tile classes."""
import numpy as np
import pytest

import oracle
import workloads
from gpu_common import build, host, say, segments_oracle

pytestmark = pytest.mark.gpu


def _check_segments(wl):
    say(f"[segments] {wl.name} T={wl.total_tokens} N={wl.total_items}")
    seg = build(wl)
    so = segments_oracle(wl)
    assert np.array_equal(host(seg.array("item_id")), so["item_id"])
    assert np.array_equal(host(seg.array("pos_id")), so["pos_id"])
    assert np.array_equal(host(seg.array("readout_pos")), so["readout_pos"])
    # each item's first token: the token after the previous readout, or the prefix end
    begin = host(seg.array("item_begin"))
    for i in range(wl.total_items):
        r = int(np.searchsorted(wl.cu_items[1:], i, side="right"))
        assert begin[i] == wl.cu_seqlens[r] + wl.item_starts[i]
    cls_o, cu_o = oracle.tile_classes(wl.cu_seqlens, so["item_id"], seg.block_m, seg.block_n)
    cls = host(seg.array("tile_class"))
    assert np.array_equal(host(seg.array("cu_tiles")), cu_o)
    assert np.array_equal(cls, cls_o)
    _check_work_list(wl, seg, cls)
    return seg


def _check_work_list(wl, seg, cls):
    """Every tile with a visible cell is visited exactly once; no empty tile is visited."""
    work = host(seg.array("work")).reshape(-1, 4)
    bm, bn = seg.block_m, seg.block_n
    cu_tiles = host(seg.array("cu_tiles"))
    seen = np.zeros(cls.shape[0], dtype=np.int64)
    costs = []
    for r, qt, a_end, b_lo in work:
        Tr = int(wl.cu_seqlens[r + 1] - wl.cu_seqlens[r])
        nkt = -(-Tr // bn)
        j1 = min(Tr, (qt + 1) * bm)
        b_hi = -(-j1 // bn)
        visit = list(range(a_end)) + list(range(max(b_lo, a_end), b_hi))
        costs.append(len(visit))
        for kt in visit:
            seen[cu_tiles[r] + qt * nkt + kt] += 1
    assert (seen <= 1).all()
    assert ((seen == 1) == (cls != 0)).all()
    # the visit count the attention dispatcher reads: every tile with a visible cell
    assert seg.struct.num_visits == int((cls != 0).sum()) == sum(costs)
    assert all(costs[i] >= costs[i + 1] for i in range(len(costs) - 1))
    assert sorted(map(tuple, work[:, :2].tolist())) == sorted(
        (r, qt) for r in range(wl.num_requests)
        for qt in range(-(-int(wl.cu_seqlens[r + 1] - wl.cu_seqlens[r]) // bm)))


@pytest.mark.parametrize("k", [1, 2, 3, 4, 5])
def test_segments_configs(k):
    _check_segments(workloads.config(k))


@pytest.mark.parametrize("seed", range(6))
def test_segments_random_shapes(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 5))
    prefix, items = [], []
    for _ in range(B):
        lq = int(rng.integers(0, 300))
        n = int(rng.integers(0 if lq else 1, 30))
        prefix.append(lq)
        items.append(rng.integers(1, 90, size=n).tolist())
    wl = workloads.from_lengths(f"rand{seed}", prefix, items, hq=8, hkv=4, d=128)
    _check_segments(wl)


def test_segments_edge_shapes():
    cases = [
        ([1], [[]]),  # single prefix token
        ([0], [[1]]),  # single one-token item
        ([0], [[1] * 70]),  # only one-token items
        ([65], [[]]),  # T = 1 mod 64: last tile holds one row
        ([64], [[1]]),
        ([63], [[1, 1]]),
        ([128], [[64, 64, 1]]),
        ([5, 0, 200], [[3], [7, 9], []]),
    ]
    for i, (p, it) in enumerate(cases):
        _check_segments(workloads.from_lengths(f"edge{i}", p, it, hq=8, hkv=4, d=128))


def test_many_builds_in_flight_keep_their_own_metadata():
    # more builds than staging slots, queued without a host sync in between
    import item_scoring_attention_amd as mis

    rng = np.random.default_rng(7)
    wls, segs = [], []
    for i in range(20):
        lq = int(rng.integers(0, 400))
        items = rng.integers(1, 60, size=int(rng.integers(1, 40))).tolist()
        wl = workloads.from_lengths(f"q{i}", [lq], [items], hq=8, hkv=4, d=128)
        bm, bn = mis.mis_attention_tile_shape(mis.MIS_BF16, 8, 4, 128)
        segs.append(mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items,
                                           wl.item_starts, bm, bn))
        wls.append(wl)
    for wl, seg in zip(wls, segs):
        so = segments_oracle(wl)
        assert np.array_equal(host(seg.array("item_id")), so["item_id"])
        assert np.array_equal(host(seg.array("readout_pos")), so["readout_pos"])
        cls, _ = oracle.tile_classes(wl.cu_seqlens, so["item_id"], seg.block_m, seg.block_n)
        assert np.array_equal(host(seg.array("tile_class")), cls)


def test_packed_batch_builds_the_packers_readout_positions():
    # the token-level packer's offsets through the GPU builder
    from item_scoring_attention_amd import build_packed_segments, pack_requests
    rng = np.random.default_rng(11)
    reqs = [(rng.integers(0, 50000, size=int(rng.integers(1, 300))),
             [rng.integers(0, 50000, size=int(rng.integers(0, 40))) for _ in range(int(rng.integers(0, 30)))])
            for _ in range(6)]
    p = pack_requests(reqs, delimiter_id=50001)
    seg = build_packed_segments(p, 64, 64)
    so = oracle.build_segments(p.cu_seqlens, p.prefix_lens, p.cu_items, p.item_starts)
    readout = host(seg.array("readout_pos"))
    assert np.array_equal(readout, so["readout_pos"])
    assert (p.token_ids[readout] == 50001).all()  # every item is read at its delimiter
    assert np.array_equal(host(seg.array("item_id")), so["item_id"])
    assert np.array_equal(host(seg.array("pos_id")), so["pos_id"])

