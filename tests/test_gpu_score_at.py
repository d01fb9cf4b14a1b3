"""Label scores at caller-chosen rows (mis_score_labels_at) vs the oracle.

Several readout markers per item (setwise scoring) and graded multi-class
labels (K = 5, with and without the softmax over the labels); at the items'
readout positions it must reproduce mis_score_labels bit for bit.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_SCORE, TOL_F32, build, dev, host, say, segments_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["auto", "narrow", "wide4", "wide6"])
def score_kernel(request):
    """Every case with the bf16 LM-head kernel chosen by shape (narrow tiles up
    to 64 items, else wide tiles with 3, 5 or 8 item blocks), and forced to the
    narrow tiles and to wide tiles of 4 and 6 item blocks."""
    mis.set_kernel_choice(score=request.param)
    yield request.param
    mis.set_kernel_choice()


def _markers(wl, so):
    """First, middle and last token of every item, plus the prefix's last token."""
    ends = np.append(wl.item_starts[1:], 0)
    pos = []
    for r in range(wl.num_requests):
        base = int(wl.cu_seqlens[r])
        a, b = int(wl.cu_items[r]), int(wl.cu_items[r + 1])
        for i in range(a, b):
            s0 = base + int(wl.item_starts[i])
            s1 = int(so["readout_pos"][i])
            pos += [s0, (s0 + s1) // 2, s1]
        if wl.prefix_lens[r] > 0:
            pos.append(base + int(wl.prefix_lens[r]) - 1)
    return np.asarray(pos, dtype=np.int32)


def _hidden(wl, rows, dtype, seed=3):
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((len(rows), wl.hidden)).astype(np.float32)
    if dtype == "bf16":
        full = np.full((wl.total_tokens, wl.hidden), workloads.NAN_BF16, dtype=np.uint16)
        full[rows] = workloads.f32_to_bf16_bits(h)
    else:
        full = np.full((wl.total_tokens, wl.hidden), np.nan, dtype=np.float32)
        full[rows] = h
    return full


@pytest.mark.parametrize("dtype,tol", [("bf16", TOL_BF16_SCORE), ("f32", TOL_F32)])
@pytest.mark.parametrize("apply_softmax", [False, True])
def test_markers_and_graded_labels(dtype, tol, apply_softmax):
    wl = workloads.from_lengths(f"markers-{dtype}", [40, 0], [[7, 1, 19, 5], [3, 12]], hq=4, hkv=2,
                                d=128 if dtype == "bf16" else 64, dtype=dtype, hidden=256, vocab=3000,
                                num_labels=5, seed=17)
    so = segments_oracle(wl)
    pos = _markers(wl, so)
    pos = np.concatenate([pos, pos[:3]])  # repeated rows are allowed
    say(f"[score_at] {wl.name} rows={len(pos)} softmax={apply_softmax}")
    hid = _hidden(wl, np.unique(pos), dtype)
    W = workloads.lm_head(wl)
    labels = workloads.label_ids(wl)
    s = mis.mis_score_labels_at(pos, dev(hid), dev(W), labels, apply_softmax=apply_softmax)
    torch.cuda.synchronize()
    ref = oracle.label_scores(hid, pos, W, labels, apply_softmax=apply_softmax)
    assert np.abs(host(s).astype(np.float64) - ref).max() <= tol


def test_readout_positions_reproduce_item_scores_bit_for_bit():
    wl = workloads.config(2)
    say(f"[score_at] {wl.name}")
    seg = build(wl)
    readout = host(seg.array("readout_pos"))
    hid = _hidden(wl, readout, "bf16")
    W = dev(workloads.lm_head(wl))
    labels = workloads.label_ids(wl)
    a = host(mis.mis_score_labels(seg, dev(hid), W, labels))
    b = host(mis.mis_score_labels_at(readout, dev(hid), W, labels))
    assert np.array_equal(a, b)


def test_no_rows():
    wl = workloads.from_lengths("markers-none", [8], [[]], hq=4, hkv=2, d=128, hidden=256, vocab=1000,
                                num_labels=2)
    hid = _hidden(wl, np.arange(1), "bf16")
    s = mis.mis_score_labels_at([], dev(hid), dev(workloads.lm_head(wl)), workloads.label_ids(wl))
    assert tuple(s.shape) == (0, 2)
