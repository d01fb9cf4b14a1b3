"""GPU label scoring vs the fp64 oracle: full-vocab log-probs, label softmax, edge cases.

Hidden rows other than the items' readout rows hold NaN, so any read of a
wrong row shows up as a NaN score.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import (TOL_BF16_SCORE, TOL_F32, build, cached, dev, hidden_with_sentinels, host, say,
                        segments_oracle)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["auto", "narrow", "wide4", "wide6", "persist3", "persist4"])
def score_kernel(request):
    """Every case with the bf16 LM-head kernel chosen by shape (narrow tiles up
    to 64 items, else the persistent wide tiles with 3, 4 or 5 item blocks),
    and forced to the narrow tiles, to the non-persistent wide tiles of 4 and 6
    item blocks and to the persistent ones of 3 and 4."""
    mis.set_kernel_choice(score=request.param)
    yield request.param
    mis.set_kernel_choice()


def _score(wl, seg, hid, W, labels, apply_softmax=False):
    hd = hid if isinstance(hid, torch.Tensor) else dev(hid)
    Wd = W if isinstance(W, torch.Tensor) else dev(W)
    s = mis.mis_score_labels(seg, hd, Wd, labels, apply_softmax=apply_softmax,
                             scores=torch.full((seg.total_items, len(labels)), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    return host(s).astype(np.float64)


def _config_case(wl):
    """Inputs (host and device) and oracle scores of a whole workload, all items."""
    so = segments_oracle(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    labels = workloads.label_ids(wl)
    say(f"  oracle: {wl.total_items} items x {wl.vocab} vocabulary rows")
    ref = oracle.label_scores(hid, so["readout_pos"], W, labels)
    refp = oracle.label_scores(hid, so["readout_pos"], W, labels, apply_softmax=True)
    return dev(hid), dev(W), labels, ref, refp


def _check_config(wl):
    tol = TOL_F32 if wl.dtype == "f32" else TOL_BF16_SCORE
    say(f"[score] {wl.name} N={wl.total_items} H={wl.hidden} V={wl.vocab} K={wl.num_labels}")
    hid, W, labels, ref, refp = cached(("score-case", wl.name), lambda: _config_case(wl))
    seg = build(wl)
    got = _score(wl, seg, hid, W, labels)
    assert np.isfinite(got).all()
    e = float(np.abs(got - ref).max())
    say(f"  logp max abs err {e:.3e} over {wl.total_items} items")
    assert e <= tol
    # log-probs are <= 0 and the label mass is at most one
    assert (got <= tol).all()
    assert (np.log(np.exp(got).sum(axis=1)) <= tol).all()
    p = _score(wl, seg, hid, W, labels, apply_softmax=True)
    assert np.isfinite(p).all()
    ep = float(np.abs(p - refp).max())
    say(f"  softmax max abs err {ep:.3e}")
    assert ep <= tol
    assert np.abs(p.sum(axis=1) - 1.0).max() <= 1e-5


def test_tiny_f32_config():
    _check_config(workloads.config(1))


def test_single_request_config():
    _check_config(workloads.config(2))


def test_profile_labeling_config():
    _check_config(workloads.config(3))


def test_long_prefix_config_every_item():
    _check_config(workloads.config(5))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("n_items,vocab", [(1, 1000), (32, 1000), (37, 129), (64, 2000), (65, 1000),
                                            (160, 700), (200, 300), (257, 300), (300, 1)])
def test_item_and_vocab_edges(dtype, n_items, vocab):
    # ragged vocabulary tiles, item tiles with a tail or exactly full (32, 64,
    # 160 = 5 x 32 items; 257 one past 8 x 32), labels at both vocabulary ends
    lens = [3] * n_items
    wl = workloads.from_lengths("edge", [10], [lens], dtype=dtype, hq=4, hkv=2, d=128, hidden=64,
                                vocab=vocab, num_labels=1)
    so = segments_oracle(wl)
    seg = build(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    labels = sorted({0, vocab - 1, vocab // 2, 0})
    got = _score(wl, seg, hid, W, labels)
    ref = oracle.label_scores(hid, so["readout_pos"], W, labels)
    tol = TOL_F32 if dtype == "f32" else TOL_BF16_SCORE
    assert np.abs(got - ref).max() <= tol
    if vocab == 1:
        assert np.abs(got).max() <= tol  # a one-word vocabulary has log-prob 0


@pytest.mark.parametrize("hidden", [128, 192])
@pytest.mark.parametrize("n_items,vocab", [(300, 120001), (97, 70000), (65, 33000), (129, 255), (70, 1)])
def test_several_tiles_per_workgroup(hidden, n_items, vocab):
    # The persistent kernel (more than 64 items, H >= 128) runs one workgroup
    # per CU, so these vocabularies give most workgroups two or three tiles
    # in a row; H = 128 and 192 make the chunk sequence cross into the next
    # tile while the ring's first chunks are still being staged. Ragged
    # vocabulary and item tails, a single partial vocabulary tile, a
    # one-word vocabulary; labels at both vocabulary ends and in the middle.
    wl = workloads.from_lengths("persist", [12], [[2] * n_items], hq=4, hkv=2, d=128, hidden=hidden,
                                vocab=vocab, num_labels=3)
    so = segments_oracle(wl)
    seg = build(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    labels = sorted({0, vocab - 1, vocab // 2, (7 * vocab) // 9})
    say(f"[score] persistent tiles N={n_items} V={vocab} H={hidden}")
    got = _score(wl, seg, hid, W, labels)
    assert np.isfinite(got).all()
    ref = oracle.label_scores(hid, so["readout_pos"], W, labels)
    assert np.abs(got - ref).max() <= TOL_BF16_SCORE
    p = _score(wl, seg, hid, W, labels, apply_softmax=True)
    refp = oracle.label_scores(hid, so["readout_pos"], W, labels, apply_softmax=True)
    assert np.abs(p - refp).max() <= TOL_BF16_SCORE


@pytest.mark.parametrize("hidden", [32, 96, 160])
@pytest.mark.parametrize("n_items,vocab", [(5, 1000), (70, 129), (200, 300)])
def test_hidden_not_a_multiple_of_64(hidden, n_items, vocab):
    # bf16 scoring with H % 64 != 0 takes the kernel that reads both operands
    # from global memory (one, two or four item blocks by N)
    wl = workloads.from_lengths("h32", [10], [[2] * n_items], hq=4, hkv=2, d=128, hidden=hidden,
                                vocab=vocab, num_labels=2)
    so = segments_oracle(wl)
    seg = build(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    labels = sorted({0, vocab - 1, vocab // 3})
    got = _score(wl, seg, hid, W, labels)
    ref = oracle.label_scores(hid, so["readout_pos"], W, labels)
    assert np.abs(got - ref).max() <= TOL_BF16_SCORE
    p = _score(wl, seg, hid, W, labels, apply_softmax=True)
    refp = oracle.label_scores(hid, so["readout_pos"], W, labels, apply_softmax=True)
    assert np.abs(p - refp).max() <= TOL_BF16_SCORE


def test_duplicate_labels_repeat_columns():
    wl = workloads.from_lengths("dup", [20], [[4] * 5], hq=4, hkv=2, d=128, hidden=128, vocab=5000,
                                num_labels=2)
    so = segments_oracle(wl)
    seg = build(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    labels = [17, 4999, 17]
    got = _score(wl, seg, hid, W, labels)
    assert np.array_equal(got[:, 0], got[:, 2])
    ref = oracle.label_scores(hid, so["readout_pos"], W, labels)
    assert np.abs(got - ref).max() <= TOL_BF16_SCORE


def test_whole_vocab_as_labels_sums_to_one():
    wl = workloads.from_lengths("all", [8], [[2] * 3], hq=4, hkv=2, d=128, hidden=64, vocab=256,
                                num_labels=1)
    so = segments_oracle(wl)
    seg = build(wl)
    hid = hidden_with_sentinels(wl, so["readout_pos"])
    W = workloads.lm_head(wl)
    got = _score(wl, seg, hid, W, list(range(256)))
    assert np.abs(np.exp(got).sum(axis=1) - 1.0).max() <= 1e-4


def test_chained_tiny_config_equals_single_item_scores():
    # hidden := MIS attention output [T, Hq*D] (Hq*D == H == 256), read at each item's last token
    wl = workloads.config(1)
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    o = mis.mis_attention_prefill(seg, dev(q), dev(k), dev(v))
    hid = o.reshape(wl.total_tokens, wl.hq * wl.d).contiguous()
    W = workloads.lm_head(wl)
    labels = workloads.label_ids(wl)
    got = host(mis.mis_score_labels(seg, hid, dev(W), labels)).astype(np.float64)
    sis = oracle.sis_scores(q, k, v, int(wl.prefix_lens[0]), wl.item_lengths().tolist(), W, labels)
    assert np.abs(got - sis).max() <= TOL_F32


def test_no_items_is_a_no_op():
    wl = workloads.from_lengths("none", [50], [[]], hq=4, hkv=2, d=128, hidden=64, vocab=100,
                                num_labels=1)
    seg = build(wl)
    hid = np.zeros((50, 64), dtype=np.uint16)
    W = workloads.lm_head(wl)
    out = mis.mis_score_labels(seg, dev(hid), dev(W), [3])
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, 1)
