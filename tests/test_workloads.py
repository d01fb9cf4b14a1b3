"""Seeded input generators: determinism, bf16 rounding, and the five workload shapes."""
import numpy as np
import pytest
import torch

import workloads


def test_bf16_rounding_matches_torch_round_to_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.standard_normal(100000).astype(np.float32),
        np.array([1.0, -2.5, 3.0039062, 1.00390625, 1.01171875, 0.0, -0.0, 65504.0], np.float32),
    ])
    ours = workloads.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(workloads.bf16_bits_to_f32(ours),
                          torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_generation_is_deterministic():
    wl = workloads.config(1)
    a = workloads.qkv(wl)
    b = workloads.qkv(wl)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert np.array_equal(workloads.lm_head(wl), workloads.lm_head(wl))
    assert np.array_equal(workloads.label_ids(wl), workloads.label_ids(wl))


def test_config_shapes():
    expect = {  # (requests, tokens, items) from the workload descriptions
        1: (1, 64 + 4 * 9, 4),
        2: (1, 2048 + 64 * 33, 64),
        5: (4, 4 * (16384 + 256 * 49), 1024),
    }
    for k, (b, t, n) in expect.items():
        wl = workloads.config(k)
        assert (wl.num_requests, wl.total_tokens, wl.total_items) == (b, t, n)
    wl3 = workloads.config(3)
    lens = wl3.item_lengths()
    assert wl3.total_items == 300 and lens.min() >= 7 and lens.max() <= 21
    wl4 = workloads.config(4)
    assert wl4.num_requests == 32
    assert wl4.prefix_lens.min() >= 512 and wl4.prefix_lens.max() <= 4096
    n_per = np.diff(wl4.cu_items)
    assert n_per.min() >= 16 and n_per.max() <= 128
    l4 = wl4.item_lengths()
    assert l4.min() >= 17 and l4.max() <= 65


def test_structure_is_contiguous():
    for k in range(1, 6):
        wl = workloads.config(k)
        for r in range(wl.num_requests):
            a, b = int(wl.cu_items[r]), int(wl.cu_items[r + 1])
            if b > a:
                assert wl.item_starts[a] == wl.prefix_lens[r]
            assert (wl.item_lengths()[a:b] >= 1).all()
            assert wl.prefix_lens[r] + wl.item_lengths()[a:b].sum() == wl.seq_len(r)


def test_labels_distinct_and_in_range():
    for k in (1, 2, 3, 5):
        wl = workloads.config(k)
        lab = workloads.label_ids(wl)
        assert len(set(lab.tolist())) == wl.num_labels
        assert lab.min() >= 0 and lab.max() < wl.vocab


def test_paper_query_lengths_match_the_quoted_statistics():
    # From Generation to Scoring, §6.1: median 543, mean 744, 95th percentile 2,047
    x = workloads.paper_query_lengths(400_000, 6)
    assert abs(np.median(x) - 543) <= 3
    assert abs(x.mean() - 744) / 744 < 0.01
    assert 1950 <= np.percentile(x, 95) <= 2050
    assert x.min() >= 1


def test_paper_query_lengths_stratified():
    x = workloads.paper_query_lengths(32, 6, stratified=True)
    assert np.median(x) == 543 and abs(x.mean() - 744) / 744 < 0.03
    assert sorted(x) == sorted(workloads.paper_query_lengths(32, 7, stratified=True))  # same quantiles
    assert not np.array_equal(x, workloads.paper_query_lengths(32, 7, stratified=True))  # another order


def test_paper_batch_request_sizes():
    # about 6,400 tokens per member at N = 200 items of 28 tokens (§6.1)
    wl = workloads.paper_batch(64, 200, 28)
    assert wl.total_items == 64 * 200
    assert np.all(wl.item_lengths() == 28)
    assert abs(wl.total_tokens / 64 - 6344) / 6344 < 0.15


def test_bench_layouts_regroup_the_same_rows():
    import bench

    wl = workloads.paper_batch(3, 200, 24)
    rows, cu, pl, ci, st = bench.layout(wl, [(r, range(200)) for r in range(3)])
    assert np.array_equal(rows, np.arange(wl.total_tokens))
    assert np.array_equal(cu, wl.cu_seqlens) and np.array_equal(st, wl.item_starts)
    rows, cu, pl, ci, st = bench.layout(wl, [(r, [i]) for r in range(3) for i in range(200)])
    assert cu[-1] == int(sum(200 * (int(lq) + 24) for lq in wl.prefix_lens))
    assert np.all(st == np.repeat(wl.prefix_lens, 200))
    # the single-item layout's prefill-token ratio is Eq. 5's R(N) summed over the batch
    assert cu[-1] / wl.total_tokens == pytest.approx(
        sum(200 * int(lq) + 200 * 24 for lq in wl.prefix_lens) / sum(int(lq) + 200 * 24 for lq in wl.prefix_lens))
