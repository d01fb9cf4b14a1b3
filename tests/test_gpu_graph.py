"""Attention and label scoring captured in a HIP graph replay to the eager
results bit for bit.

The attention and scoring calls enqueue kernels only (no memory sets, copies
or host waits), so a caller can capture them once a segment buffer has been
built outside the capture. The graph is replayed several times with other
eager work and synchronisations in between, and its outputs are filled with
NaN before each replay, so every replay has to write them again.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import workloads
from gpu_common import build, dev, hidden_with_sentinels, host, say, segments_oracle

pytestmark = pytest.mark.gpu

REPLAYS = 3


def _workload(name):
    if name == "single-request":
        return workloads.config(2)  # 64 items: the narrow scoring tiles
    # 290 items: the persistent scoring workgroups
    return workloads.from_lengths("graph-persist", [500, 200], [[12] * 150, [7] * 140], hq=8, hkv=4, d=128,
                                  hidden=1024, vocab=50000, num_labels=3, seed=51)


@pytest.mark.parametrize("name", ["single-request", "persistent-scoring"])
def test_captured_attention_and_scoring_replay_the_eager_results(name):
    wl = _workload(name)
    say(f"[graph] {wl.name} T={wl.total_tokens} N={wl.total_items}")
    q, k, v = workloads.qkv(wl)
    qd, kd, vd = dev(q), dev(k), dev(v)
    so = segments_oracle(wl)
    hid = dev(hidden_with_sentinels(wl, so["readout_pos"]))
    W = dev(workloads.lm_head(wl))
    labels = workloads.label_ids(wl)
    seg = build(wl)  # outside the capture: its metadata upload is a host copy
    N, K = wl.total_items, len(labels)
    ws = torch.empty(mis.mis_score_workspace_bytes(N, wl.vocab, K, wl.hidden, mis.MIS_BF16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty_like(qd)
    scores = torch.empty((N, K), dtype=torch.float32, device="cuda")
    scores_na = torch.empty((N, K), dtype=torch.float32, device="cuda")

    def calls():
        mis.mis_attention_prefill(seg, qd, kd, vd, o=o)
        mis.mis_score_labels(seg, hid, W, labels, scores=scores, ws=ws)
        mis.mis_score_labels_noalloc(seg, hid, W, labels, scores=scores_na)

    def outputs():
        return host(o), host(scores), host(scores_na)

    def clear():
        o.fill_(float("nan"))
        scores.fill_(float("nan"))
        scores_na.fill_(float("nan"))

    clear()
    calls()
    torch.cuda.synchronize()
    want = outputs()
    assert np.isfinite(want[1]).all() and np.array_equal(want[1], want[2])

    side = torch.cuda.Stream()  # default priority
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        calls()  # warm-up on the capture stream, as torch recommends
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        calls()
    torch.cuda.synchronize()

    other = torch.empty_like(qd)
    for r in range(REPLAYS):
        clear()
        # eager work between replays: the same kernels on another output
        mis.mis_attention_prefill(seg, qd, kd, vd, o=other)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = outputs()
        for g, w, what in zip(got, want, ("attention", "scores", "allocation-free scores")):
            assert np.array_equal(g, w), f"replay {r}: {what} differ from the eager call"
    assert np.array_equal(host(other), want[0])
