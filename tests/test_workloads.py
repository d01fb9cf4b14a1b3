"""Seeded input generators: determinism, bf16 rounding, and the five workload shapes."""
import numpy as np
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
