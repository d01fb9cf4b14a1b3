"""mis_score_labels_noalloc (the library's own per-GPU scratch, no workspace
argument) against mis_score_labels with a caller workspace, through the C ABI.

Two calls in a row, the second with fewer items and a different vocabulary,
so the second reuses the scratch the first left behind; each must equal the
workspace call bit for bit (same kernels, same partials) and the fp64 oracle
within the label log-prob tolerance.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_SCORE, build, dev, hidden_with_sentinels, host, say, segments_oracle

pytestmark = pytest.mark.gpu


def _case(wl, apply_softmax):
    so = segments_oracle(wl)
    seg = build(wl)
    hid = dev(hidden_with_sentinels(wl, so["readout_pos"]))
    W = workloads.lm_head(wl)
    Wd = dev(W)
    labels = workloads.label_ids(wl)
    N, K = wl.total_items, wl.num_labels
    a = torch.full((N, K), float("nan"), device="cuda")
    b = torch.full((N, K), float("nan"), device="cuda")
    mis.mis_score_labels(seg, hid, Wd, labels, apply_softmax=apply_softmax, scores=a)
    mis.mis_score_labels_noalloc(seg, hid, Wd, labels, apply_softmax=apply_softmax, scores=b)
    torch.cuda.synchronize()
    got_a, got_b = host(a).astype(np.float64), host(b).astype(np.float64)
    assert np.isfinite(got_b).all()
    assert np.array_equal(got_a, got_b)
    ref = oracle.label_scores(host(hid), so["readout_pos"], W, labels, apply_softmax=apply_softmax)
    e = float(np.abs(got_b - ref).max())
    say(f"[noalloc] N={N} V={wl.vocab} H={wl.hidden} softmax={apply_softmax}: max abs err {e:.3e}")
    assert e <= TOL_BF16_SCORE


@pytest.mark.parametrize("apply_softmax", [False, True])
def test_noalloc_equals_workspace_call_twice_second_smaller(apply_softmax):
    first = workloads.from_lengths("noalloc-1", [500, 200], [[12] * 150, [7] * 140], hq=8, hkv=4, d=128,
                                   hidden=1024, vocab=50000, num_labels=3, seed=31)
    second = workloads.from_lengths("noalloc-2", [300], [[9] * 40], hq=8, hkv=4, d=128, hidden=512,
                                    vocab=20000, num_labels=2, seed=32)
    _case(first, apply_softmax)
    _case(second, apply_softmax)


def test_noalloc_rejects_a_call_beyond_its_scratch():
    # 2 * N * ceil(V / 128) floats of partials above 16 MiB
    wl = workloads.from_lengths("noalloc-big", [10], [[1] * 2000], hq=4, hkv=2, d=128, hidden=64,
                                vocab=151936, num_labels=2)
    seg = build(wl)
    hid = torch.zeros((wl.total_tokens, 64), dtype=torch.bfloat16, device="cuda")
    W = torch.zeros((wl.vocab, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mis.MisError, match="MIS_ERR_WORKSPACE"):
        mis.mis_score_labels_noalloc(seg, hid, W, [1, 2])
