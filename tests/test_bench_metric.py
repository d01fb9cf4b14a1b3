"""The headline metric's work count: bench.py's unmasked (query, key) pairs,
which set the attention FLOPs of every bench line, against a count of the
visible cells of the oracle's explicit Eq. 4 mask (From Generation to
Scoring, §4.1), request by request. CPU only.
"""
import numpy as np
import pytest

import bench
import oracle
import workloads


def _mask_pairs(wl) -> int:
    so = oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    ids = so["item_id"]
    total = 0
    for r in range(wl.num_requests):
        a, b = int(wl.cu_seqlens[r]), int(wl.cu_seqlens[r + 1])
        total += oracle.visible_pairs(ids[a:b])
    return total


@pytest.mark.parametrize("prefix,items", [
    ([64], [[9, 9, 9, 9]]),
    ([0, 37, 5], [[4, 1], [12, 3, 7], []]),
    ([130, 1], [[1] * 20, [2, 2]]),
])
def test_bench_pairs_equal_the_mask(prefix, items):
    wl = workloads.from_lengths("pairs", prefix, items, hq=4, hkv=2, d=64)
    assert bench.visible_pairs(wl) == _mask_pairs(wl)


@pytest.mark.parametrize("prefix,items", [
    ([64], [[9, 9, 9, 9]]),
    ([0, 37, 5], [[4, 1], [12, 3, 7], []]),
    ([130, 1], [[1] * 20, [2, 2]]),
])
def test_append_pairs_are_the_item_rows_of_the_mask(prefix, items):
    # the work of appending items to a cached prefix: the visible cells of
    # the item rows of the explicit mask, prefix rows left out
    wl = workloads.from_lengths("pairs", prefix, items, hq=4, hkv=2, d=64)
    so = oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    ids = so["item_id"]
    want = 0
    for r in range(wl.num_requests):
        a, b = int(wl.cu_seqlens[r]), int(wl.cu_seqlens[r + 1])
        m = oracle.mis_mask(ids[a:b])
        want += int(np.count_nonzero(m[ids[a:b] >= 0] == 0.0))
    assert bench.visible_pairs(wl, items_only=True) == want
    assert bench.attention_flops(wl, items_only=True) == 4 * 64 * 4 * want


def test_tiny_workload_pairs_and_flops():
    wl = workloads.config(1)
    assert bench.visible_pairs(wl) == _mask_pairs(wl)
    assert bench.attention_flops(wl) == 4 * wl.d * wl.hq * _mask_pairs(wl)


def test_single_request_workload_figures():
    # prefix 2048 + 64 items of 33 tokens, 16 query heads of 128 dims
    wl = workloads.config(2)
    lq, s, n = 2048, 33, 64
    pairs = lq * (lq + 1) // 2 + n * (s * lq + s * (s + 1) // 2)
    assert pairs == 6_459_456
    assert bench.visible_pairs(wl) == pairs
    assert bench.attention_flops(wl) == 4 * 128 * 16 * pairs == 52_915_863_552


def test_single_request_scoring_figures():
    # 64 items, H = 1024, V = 151936, K = 2: FLOPs 2NHV; bytes: the LM head and
    # the readout rows read once (bf16), the label log-probs written (fp32)
    wl = workloads.config(2)
    flops, nbytes = bench.lm_head_cost(wl)
    assert flops == 2 * 64 * 1024 * 151936 == 19_914_555_392
    assert nbytes == 2 * (151936 * 1024 + 64 * 1024) + 4 * 64 * 2 == 311_296_512


def test_long_prefix_workload_figures():
    # 4 requests: prefix 16384 + 256 items of 49 tokens, 64 query heads of 128
    # dims; scoring H = 8192, V = 128256, K = 3 (the bench's default workload)
    wl = workloads.config(5)
    lq, s, n = 16384, 49, 256
    pairs = 4 * (lq * (lq + 1) // 2 + n * (s * lq + s * (s + 1) // 2))
    assert pairs == 1_360_241_664
    assert bench.visible_pairs(wl) == pairs
    assert bench.attention_flops(wl) == 4 * 128 * 64 * pairs == 44_572_398_845_952
    flops, nbytes = bench.lm_head_cost(wl)
    assert flops == 2 * 1024 * 8192 * 128256 == 2_151_778_615_296
    assert nbytes == 2 * (128256 * 8192 + 1024 * 8192) + 4 * 1024 * 3
