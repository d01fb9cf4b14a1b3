"""Seeded synthetic inputs for multiple-item scoring (MIS).

This module is shared by the tests, the benchmark and the smoke check. It
only draws random structure (prefix lengths, item counts, item lengths) and
random values (Q/K/V, readout hidden rows, LM head, label ids). It holds none
of the method's arithmetic: no masks, no positions, no attention, no softmax.
Both the fp64 oracle and the HIP library receive exactly the bytes made here.

Workload shapes follow the pages' setting of one long shared prefix followed
by tens to hundreds of short candidate items (From Generation to Scoring,
§2.2 workload shape and §6.1 benchmark; LinkedIn SGLang blog, Results
section: 12K-token prefix with 50 items of 150 tokens). The proprietary
profile set and the Open-Jev dataset are not reproduced; these seeded
generators stand in for them.

Layout conventions (request-major packed "varlen"):

* ``cu_seqlens[B+1]``: token offsets of the requests in the packed sequence.
* ``prefix_lens[B]``: shared-prefix length Lq of each request.
* ``cu_items[B+1]``: offsets of each request's items in the global item list.
* ``item_starts[N]``: request-relative first token of every item. Every item
  is its content tokens followed by one closing delimiter token, and the
  items of a request tile ``[Lq, T_r)`` contiguously in input order.

Values: Q/K/V ~ N(0,1), LM head ~ N(0, 0.02), readout hidden rows ~ N(0,1),
label ids distinct and uniform in ``[0, V)``. Floating-point values are drawn
in float32 and, for bf16 workloads, rounded to bf16 with round-to-nearest-even
so that both sides see the same bits.
"""
from __future__ import annotations

import concurrent.futures as _cf
import dataclasses
import os
from typing import List, Optional, Sequence

import numpy as np

__all__ = [
    "Workload",
    "CONFIGS",
    "config",
    "from_lengths",
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "qkv",
    "readout_values",
    "lm_head",
    "label_ids",
    "NAN_BF16",
    "PAPER_QUERY_MEDIAN",
    "PAPER_QUERY_MEAN",
    "paper_query_lengths",
    "paper_batch",
]

# Quiet-NaN bit pattern in bf16 (sign 0, exponent all ones, mantissa 0x40).
NAN_BF16 = np.uint16(0x7FC0)

# Child-stream order of SeedSequence(seed).spawn(...): never reorder.
_STREAMS = ("structure", "q", "k", "v", "hidden", "lm_head", "labels")


@dataclasses.dataclass
class Workload:
    """One synthetic MIS batch: packed structure plus shape parameters."""

    name: str
    seed: int
    dtype: str  # "f32" or "bf16"
    hq: int
    hkv: int
    d: int
    cu_seqlens: np.ndarray
    prefix_lens: np.ndarray
    cu_items: np.ndarray
    item_starts: np.ndarray
    hidden: Optional[int] = None  # label-scoring hidden size H
    vocab: Optional[int] = None  # V
    num_labels: Optional[int] = None  # K
    lm_std: float = 0.02
    description: str = ""

    @property
    def num_requests(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def total_items(self) -> int:
        return int(self.cu_items[-1])

    @property
    def has_scoring(self) -> bool:
        return self.hidden is not None

    def seq_len(self, r: int) -> int:
        return int(self.cu_seqlens[r + 1] - self.cu_seqlens[r])

    def item_lengths(self) -> np.ndarray:
        """Token count of every item (content plus its closing delimiter)."""
        out = np.empty(self.total_items, dtype=np.int64)
        for r in range(self.num_requests):
            a, b = int(self.cu_items[r]), int(self.cu_items[r + 1])
            ends = np.append(self.item_starts[a + 1 : b], self.seq_len(r))
            out[a:b] = ends - self.item_starts[a:b]
        return out

    def _streams(self):
        return dict(zip(_STREAMS, np.random.SeedSequence(self.seed).spawn(len(_STREAMS))))


def from_lengths(
    name: str,
    prefix_lens: Sequence[int],
    item_lens: Sequence[Sequence[int]],
    *,
    seed: int = 0,
    dtype: str = "bf16",
    hq: int = 4,
    hkv: int = 2,
    d: int = 128,
    hidden: Optional[int] = None,
    vocab: Optional[int] = None,
    num_labels: Optional[int] = None,
    description: str = "",
) -> Workload:
    """Lay out requests from a prefix length and item token counts per request.

    ``item_lens[r][i]`` counts the item's tokens including its closing
    delimiter. Items follow the prefix back to back in the given order.
    """
    if len(prefix_lens) != len(item_lens):
        raise ValueError("prefix_lens and item_lens differ in length")
    cu_seqlens = [0]
    cu_items = [0]
    starts: List[int] = []
    for lq, lens in zip(prefix_lens, item_lens):
        off = int(lq)
        for s in lens:
            starts.append(off)
            off += int(s)
        cu_seqlens.append(cu_seqlens[-1] + off)
        cu_items.append(cu_items[-1] + len(lens))
    return Workload(
        name=name,
        seed=seed,
        dtype=dtype,
        hq=hq,
        hkv=hkv,
        d=d,
        cu_seqlens=np.asarray(cu_seqlens, dtype=np.int32),
        prefix_lens=np.asarray(prefix_lens, dtype=np.int32),
        cu_items=np.asarray(cu_items, dtype=np.int32),
        item_starts=np.asarray(starts, dtype=np.int32),
        hidden=hidden,
        vocab=vocab,
        num_labels=num_labels,
        description=description,
    )


def _cfg1() -> Workload:
    return from_lengths(
        "tiny-f32", [64], [[9] * 4], seed=1, dtype="f32", hq=4, hkv=4, d=64,
        hidden=256, vocab=1000, num_labels=2,
        description="1 request, prefix 64 + 4 items x (8+1 delimiter), MHA 4 heads, "
        "head_dim 64, fp32; scoring H=256 V=1000 K=2",
    )


def _cfg2() -> Workload:
    return from_lengths(
        "single-request-bf16", [2048], [[33] * 64], seed=2, dtype="bf16", hq=16, hkv=8,
        d=128, hidden=1024, vocab=151936, num_labels=2,
        description="1 request, prefix 2048 + 64 items x (32+1), GQA 16q/8kv, head_dim 128, "
        "bf16; scoring H=1024 V=151936 K=2",
    )


def _cfg3() -> Workload:
    rng = np.random.default_rng(np.random.SeedSequence(3).spawn(len(_STREAMS))[0])
    lens = (rng.integers(6, 21, size=300) + 1).tolist()
    return from_lengths(
        "profile-labeling-bf16", [1536], [lens], seed=3, dtype="bf16", hq=32, hkv=8,
        d=128, hidden=4096, vocab=151936, num_labels=2,
        description="1 request, prefix 1536 + 300 items of U{6..20}+1 tokens, GQA 32q/8kv, "
        "head_dim 128, bf16; scoring H=4096 V=151936 K=2",
    )


def _cfg4() -> Workload:
    rng = np.random.default_rng(np.random.SeedSequence(4).spawn(len(_STREAMS))[0])
    prefix, items = [], []
    for _ in range(32):
        prefix.append(int(rng.integers(512, 4097)))
        n = int(rng.integers(16, 129))
        items.append((rng.integers(16, 65, size=n) + 1).tolist())
    return from_lengths(
        "ragged-serving-bf16", prefix, items, seed=4, dtype="bf16", hq=32, hkv=8, d=128,
        description="32 requests, prefix U{512..4096}, U{16..128} items of U{16..64}+1 "
        "tokens, GQA 32q/8kv, head_dim 128, bf16; attention only",
    )


def _cfg5() -> Workload:
    return from_lengths(
        "long-prefix-bf16", [16384] * 4, [[49] * 256] * 4, seed=5, dtype="bf16", hq=64,
        hkv=8, d=128, hidden=8192, vocab=128256, num_labels=3,
        description="4 requests, prefix 16384 + 256 items x (48+1), GQA 64q/8kv, head_dim "
        "128, bf16; scoring H=8192 V=128256 K=3",
    )


CONFIGS = {1: _cfg1, 2: _cfg2, 3: _cfg3, 4: _cfg4, 5: _cfg5}


# --------------------------------------------------------------------------
# the profile-labeling benchmark's shape (From Generation to Scoring, §6.1
# "Workload": queries average 744 tokens with median 543 and 95th percentile
# 2,047; items average 28 tokens in the chat layout, about 24 in the compact
# readout-token layout of §3.1; 200 candidates per member)
# --------------------------------------------------------------------------

PAPER_QUERY_MEDIAN = 543
PAPER_QUERY_MEAN = 744


def paper_query_lengths(n: int, seed: int, stratified: bool = False) -> np.ndarray:
    """``n`` query lengths from a lognormal with the benchmark's median and
    mean: mu = ln(median), sigma^2 = 2 ln(mean / median) (its 95th percentile
    is then about 2,003 tokens against the quoted 2,047), rounded to whole
    tokens, at least 1. ``stratified``: the lognormal's quantiles at
    (i + 0.5) / n in a seeded random order, so that a batch of a few dozen
    members already has the distribution's median and nearly its mean (a
    random draw of 16 from this heavy tail can miss the mean by a third)."""
    from scipy.special import ndtri

    mu = np.log(PAPER_QUERY_MEDIAN)
    sigma = np.sqrt(2.0 * np.log(PAPER_QUERY_MEAN / PAPER_QUERY_MEDIAN))
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(len(_STREAMS))[0])
    if stratified:
        x = rng.permutation(np.exp(mu + sigma * ndtri((np.arange(n) + 0.5) / n)))
    else:
        x = rng.lognormal(mu, sigma, size=n)
    return np.maximum(1, np.rint(x)).astype(np.int64)


def paper_batch(num_members: int, items_per_member: int = 200, item_tokens: int = 28, *, seed: int = 6,
                hq: int = 16, hkv: int = 8, d: int = 128, hidden: int = 1024, vocab: int = 151936,
                num_labels: int = 2, name: str = "") -> Workload:
    """A batch of members, each one request: a query length from
    ``paper_query_lengths`` (stratified) and ``items_per_member`` items of ``item_tokens``
    tokens each (28: chat layout, 24: compact layout; the count includes the
    item's last token, where its label logits are read). The model shape
    defaults to the single-request workload's (GQA 16/8, head_dim 128, hidden
    1024, vocabulary 151936)."""
    lq = paper_query_lengths(num_members, seed, stratified=True)
    return from_lengths(
        name or f"paper-{num_members}x{items_per_member}x{item_tokens}", lq.tolist(),
        [[item_tokens] * items_per_member] * num_members, seed=seed, dtype="bf16", hq=hq, hkv=hkv, d=d,
        hidden=hidden, vocab=vocab, num_labels=num_labels,
        description=f"{num_members} members, query lengths at lognormal(median 543, mean 744) quantiles, "
        f"{items_per_member} items of "
        f"{item_tokens} tokens, GQA {hq}/{hkv}, head_dim {d}, bf16; scoring H={hidden} V={vocab} K={num_labels}",
    )


def config(k: int) -> Workload:
    """Workload ``k`` (1..5)."""
    return CONFIGS[k]()


# --------------------------------------------------------------------------
# value generation
# --------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bf16 (round to nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    out = r.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = NAN_BF16
    return out


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


_CHUNK = 1 << 22  # values per generator child stream


def _normal(ss: np.random.SeedSequence, n: int, std: float, dtype: str) -> np.ndarray:
    """``n`` N(0, std^2) values, bf16 bits (uint16) or float32.

    The count is split into fixed-size chunks with one spawned child stream
    each, so the bytes do not depend on the number of worker threads.
    """
    nchunks = max(1, -(-n // _CHUNK))
    kids = ss.spawn(nchunks)
    out = np.empty(n, dtype=np.uint16 if dtype == "bf16" else np.float32)

    def fill(i: int) -> None:
        a = i * _CHUNK
        b = min(n, a + _CHUNK)
        v = np.random.default_rng(kids[i]).standard_normal(b - a, dtype=np.float32)
        if std != 1.0:
            v *= np.float32(std)
        out[a:b] = f32_to_bf16_bits(v) if dtype == "bf16" else v

    workers = min(nchunks, max(1, min(16, os.cpu_count() or 1)))
    if workers == 1:
        for i in range(nchunks):
            fill(i)
    else:
        with _cf.ThreadPoolExecutor(workers) as ex:
            list(ex.map(fill, range(nchunks)))
    return out


def qkv(wl: Workload, scale_q: float = 1.0):
    """Q ``[T,Hq,D]``, K and V ``[T,Hkv,D]`` (bf16 bits or float32).

    ``scale_q`` multiplies Q before rounding; a value above one sharpens the
    softmax (stress input).
    """
    s = wl._streams()
    t = wl.total_tokens
    q = _normal(s["q"], t * wl.hq * wl.d, scale_q, wl.dtype).reshape(t, wl.hq, wl.d)
    k = _normal(s["k"], t * wl.hkv * wl.d, 1.0, wl.dtype).reshape(t, wl.hkv, wl.d)
    v = _normal(s["v"], t * wl.hkv * wl.d, 1.0, wl.dtype).reshape(t, wl.hkv, wl.d)
    return q, k, v


def readout_values(wl: Workload) -> np.ndarray:
    """Hidden-state rows ``[N, H]`` for the items' readout tokens, N(0,1).

    The caller places row ``n`` at item ``n``'s readout token of a ``[T, H]``
    hidden tensor whose other rows it fills with NaN.
    """
    s = wl._streams()
    return _normal(s["hidden"], wl.total_items * wl.hidden, 1.0, wl.dtype).reshape(
        wl.total_items, wl.hidden
    )


def lm_head(wl: Workload) -> np.ndarray:
    """LM head ``[V, H]`` ~ N(0, lm_std^2)."""
    s = wl._streams()
    return _normal(s["lm_head"], wl.vocab * wl.hidden, wl.lm_std, wl.dtype).reshape(
        wl.vocab, wl.hidden
    )


def label_ids(wl: Workload) -> np.ndarray:
    """``K`` distinct label token ids, uniform in ``[0, V)``."""
    rng = np.random.default_rng(wl._streams()["labels"])
    return rng.choice(wl.vocab, size=wl.num_labels, replace=False).astype(np.int32)
