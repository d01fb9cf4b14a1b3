"""Calls on two streams at once, and from two host threads, give the same bits
as the same calls one after the other.

Every call of the boundary is ordered on the stream it is given and keeps no
state between calls beyond the thread-local error text and kernel choice
(the allocation-free scoring entry, which shares one scratch array per GPU,
is not used here). One workload's metadata travels in the builder's kernel
arguments, the other's through the pinned staging ring, so both upload paths
run concurrently.
"""
import threading

import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import dev, hidden_with_sentinels, host, say, segments_oracle

pytestmark = pytest.mark.gpu

REPEATS = 3


class Case:
    """Device inputs and caller-owned outputs of one workload's step."""

    def __init__(self, wl):
        self.wl = wl
        self.dt = mis.MIS_BF16
        self.bm, self.bn = mis.mis_attention_tile_shape(self.dt, wl.hq, wl.hkv, wl.d)
        q, k, v = workloads.qkv(wl)
        self.q, self.k, self.v = dev(q), dev(k), dev(v)
        so = segments_oracle(wl)
        self.hid = dev(hidden_with_sentinels(wl, so["readout_pos"]))
        self.W = dev(workloads.lm_head(wl))
        self.labels = workloads.label_ids(wl)
        N = wl.total_items
        self.seg_buf = torch.empty(mis.mis_segments_bytes(wl.cu_seqlens, N, self.bm, self.bn), dtype=torch.uint8,
                                   device="cuda")
        self.ws = torch.empty(mis.mis_score_workspace_bytes(N, wl.vocab, len(self.labels), wl.hidden, self.dt),
                              dtype=torch.uint8, device="cuda")
        self.o = torch.empty_like(self.q)
        self.scores = torch.empty((N, len(self.labels)), dtype=torch.float32, device="cuda")

    def reset(self):
        self.o.fill_(float("nan"))
        self.scores.fill_(float("nan"))

    def step(self, stream):
        wl = self.wl
        s = mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, self.bm, self.bn,
                                   dev_buf=self.seg_buf, stream=stream)
        mis.mis_attention_prefill(s, self.q, self.k, self.v, o=self.o, stream=stream)
        mis.mis_score_labels(s, self.hid, self.W, self.labels, scores=self.scores, ws=self.ws, stream=stream)

    def result(self):
        return host(self.o), host(self.scores)


def _cases():
    a = workloads.config(2)  # metadata small enough for the builder's kernel arguments
    rng = np.random.default_rng(41)
    b = workloads.from_lengths("streams-ring", [int(x) for x in rng.integers(100, 900, 12)],
                               [[int(x) for x in rng.integers(3, 20, 70)] for _ in range(12)],
                               hq=16, hkv=8, d=128, hidden=512, vocab=20000, num_labels=3, seed=42)
    assert b.total_items + len(b.cu_seqlens) > 768  # staged through the pinned ring
    return Case(a), Case(b)


def _finite(result):
    o, scores = result
    return np.isfinite(oracle.as_f64(o)).all() and np.isfinite(scores).all()


def _same(name, got, want):
    assert _finite(got), f"{name}: an output was not written"
    for g, w, what in zip(got, want, ("attention", "scores")):
        assert np.array_equal(g, w), f"{name}: {what} differ from the sequential run"


def test_two_streams_and_two_threads_match_sequential():
    A, B = _cases()
    say(f"[streams] {A.wl.name} T={A.wl.total_tokens} + {B.wl.name} T={B.wl.total_tokens} N={B.wl.total_items}")
    default = torch.cuda.current_stream()
    want = []
    for c in (A, B):
        c.reset()
        c.step(default)
        torch.cuda.synchronize()
        want.append(c.result())
        assert _finite(want[-1]), f"{c.wl.name}: an output was not written"

    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()  # default priority
    for c in (A, B):
        c.reset()
    torch.cuda.synchronize()
    for _ in range(REPEATS):  # interleaved launches on two streams
        A.step(s1)
        B.step(s2)
    torch.cuda.synchronize()
    _same("two streams, A", A.result(), want[0])
    _same("two streams, B", B.result(), want[1])

    for c in (A, B):
        c.reset()
    torch.cuda.synchronize()
    errors = []

    def worker(c, st):
        try:
            with torch.cuda.stream(st):
                for _ in range(REPEATS):
                    c.step(st)
            st.synchronize()
        except Exception as e:  # reported on the main thread
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(A, s1)), threading.Thread(target=worker, args=(B, s2))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a host thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    _same("two threads, A", A.result(), want[0])
    _same("two threads, B", B.result(), want[1])
