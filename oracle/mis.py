"""Plain fp64 CPU oracle for multiple-item scoring (MIS).

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
link this module: only the test suite, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library; the two
meet only in the seeded inputs that ``workloads`` draws.

What it computes, from the pages' own statement of the method:

* Segments. One packed sequence is a shared prefix q followed by the items
  c_1..c_N (From Generation to Scoring, §4.1, Eq. 3). Position ids restart
  after the prefix in every item: prefix token u gets u, the token at offset
  d inside any item gets Lq + d (same section, position-id rule). The
  LinkedIn SGLang blog ("Multi-item-scoring" section) closes each item with a
  delimiter token; here that delimiter is the item's last token, part of
  the item's own segment, and the item's label logits are read there.
* Mask. The additive mask of Eq. 4: a token j may attend to k if k <= j and k
  lies in the prefix set Q, or if k <= j and both lie in the same item set
  I_i; every other pair gets -inf. It is built literally, as a dense matrix.
* Attention. softmax(scale * Q K^T + M) V per query head in fp64, with dense
  rows and the explicit mask; query head h reads KV head floor(h*Hkv/Hq).
* Scores. The readout hidden row of each item is projected onto the whole
  vocabulary and normalised over all of it (Scaling JEV-like Decision Models
  with SGLang, "Why a Decision Workload Deserves a Scoring Interface": label
  selection does not remove the full projection or normalisation). The
  label columns of the log-softmax come back in the requested label order.
  With ``apply_softmax`` the K label logits are renormalised among
  themselves (Eq. 2 of From Generation to Scoring for the YES/NO pair; the Score API's
  apply_softmax flag in the JEV post).
* SIS. Single-item scoring runs every [q; c_i] alone under an ordinary
  causal mask; MIS must give the same item rows and scores (From Generation to Scoring, §4.1: the
  mask and reused positions give the item's last token the context it has
  in [q; c_i]; Table 1's release check).
* Rotary embedding (the step before attention). The pages fix the positions
  only (§4.1's position-id rule). The rotation is the usual rotary position
  embedding of the decoder families the pages use: dims i and i + D/2 form a
  pair turned by the angle pos * theta^(-2i/D). With it, MIS at the reused
  positions must equal SIS at ordinary positions 0 .. Lq + S_i - 1.

Readings where the pages are silent: softmax scale 1/sqrt(D) unless given;
contiguous GQA groups; tile classes count in-range cells only (0 = no
visible cell, 1 = some, 2 = all). Row blocks below only bound memory: every
softmax row is still computed whole and independently.
"""
from __future__ import annotations

import concurrent.futures as _cf
import math
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf

# --------------------------------------------------------------------------
# input decoding (bf16 bits or float arrays -> exact float64)
# --------------------------------------------------------------------------


def as_f64(x: np.ndarray) -> np.ndarray:
    """Exact float64 value of an array of float32/float64 or of bf16 bit patterns (uint16)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


# --------------------------------------------------------------------------
# segments (From Generation to Scoring, §4.1, Eq. 3 and the position-id rule; blog's delimiter format)
# --------------------------------------------------------------------------


def build_segments(
    cu_seqlens: Sequence[int],
    prefix_lens: Sequence[int],
    cu_items: Sequence[int],
    item_starts: Sequence[int],
) -> Dict[str, np.ndarray]:
    """Per-token item id and position id, per-item readout position.

    ``item_id[t]`` is -1 for prefix tokens and the global item index
    otherwise; ``pos_id[t]`` is the reused position id; ``readout_pos[n]`` is
    the packed index of item n's last token (its closing delimiter).
    """
    cu_seqlens = [int(x) for x in cu_seqlens]
    cu_items = [int(x) for x in cu_items]
    T = cu_seqlens[-1]
    item_id = np.full(T, -2, dtype=np.int64)
    pos_id = np.full(T, -1, dtype=np.int64)
    readout = np.full(cu_items[-1], -1, dtype=np.int64)
    for r in range(len(prefix_lens)):
        base, end = cu_seqlens[r], cu_seqlens[r + 1]
        lq = int(prefix_lens[r])
        for u in range(lq):  # query tokens: positions 0..Lq-1
            item_id[base + u] = -1
            pos_id[base + u] = u
        for i in range(cu_items[r], cu_items[r + 1]):
            start = int(item_starts[i])
            stop = int(item_starts[i + 1]) if i + 1 < cu_items[r + 1] else end - base
            for d in range(stop - start):  # offset d inside the item -> Lq + d
                item_id[base + start + d] = i
                pos_id[base + start + d] = lq + d
            readout[i] = base + stop - 1
    if (item_id == -2).any():
        raise ValueError("segments do not cover every token")
    return {"item_id": item_id, "pos_id": pos_id, "readout_pos": readout}


def request_item_ids(seg: Dict[str, np.ndarray], cu_seqlens, r: int) -> np.ndarray:
    return seg["item_id"][int(cu_seqlens[r]) : int(cu_seqlens[r + 1])]


# --------------------------------------------------------------------------
# mask (From Generation to Scoring, §4.1, Eq. 4)
# --------------------------------------------------------------------------


def mis_mask(item_id_r: np.ndarray) -> np.ndarray:
    """Additive mask of one request, ``[T_r, T_r]``: 0 where attention is allowed, -inf elsewhere.

    Case 1: k <= j and k in the prefix set Q. Case 2: k <= j and j, k in the
    same item set I_i. Otherwise -inf.
    """
    ids = np.asarray(item_id_r)
    return mask_rows(ids, np.arange(ids.shape[0]))


def mask_rows(ids: np.ndarray, rows: np.ndarray) -> np.ndarray:
    """Rows ``rows`` (request-local query indices) of the Eq. 4 mask, ``[len(rows), T_r]``."""
    ids = np.asarray(ids)
    rows = np.asarray(rows, dtype=np.int64)
    T = ids.shape[0]
    j = rows[:, None]
    k = np.arange(T)[None, :]
    causal = k <= j
    k_in_query = (ids == -1)[None, :]
    j_ids = ids[rows][:, None]
    same_item = (j_ids == ids[None, :]) & (j_ids >= 0)
    allowed = (causal & k_in_query) | (causal & same_item)
    m = np.full((rows.shape[0], T), NEG_INF)
    m[allowed] = 0.0
    return m


def visible_pairs(item_id_r: np.ndarray) -> int:
    """Number of (query, key) pairs the mask lets through in one request."""
    return int(np.count_nonzero(mis_mask(item_id_r) == 0.0))


# --------------------------------------------------------------------------
# tile classes (brute force over the explicit mask)
# --------------------------------------------------------------------------


def tile_classes(
    cu_seqlens: Sequence[int], item_id: np.ndarray, block_m: int, block_n: int
) -> Tuple[np.ndarray, np.ndarray]:
    """Class of every ``block_m x block_n`` tile of every request.

    Tiles are numbered request by request, query tile major. A tile's class
    is 0 if none of its in-range cells is visible, 2 if all are, 1 otherwise.
    Returns ``(classes int8, cu_tiles int64[B+1])``.
    """
    out = []
    cu_tiles = [0]
    for r in range(len(cu_seqlens) - 1):
        ids = np.asarray(item_id[int(cu_seqlens[r]) : int(cu_seqlens[r + 1])])
        T = ids.shape[0]
        nqt = -(-T // block_m)
        nkt = -(-T // block_n)
        for qt in range(nqt):
            rows = np.arange(qt * block_m, min(T, (qt + 1) * block_m))
            vis = mask_rows(ids, rows) == 0.0  # one strip of the explicit mask
            for kt in range(nkt):
                blk = vis[:, kt * block_n : (kt + 1) * block_n]
                n_vis = int(blk.sum())
                out.append(0 if n_vis == 0 else (2 if n_vis == blk.size else 1))
        cu_tiles.append(cu_tiles[-1] + nqt * nkt)
    return np.asarray(out, dtype=np.int8), np.asarray(cu_tiles, dtype=np.int64)


# --------------------------------------------------------------------------
# attention (dense explicit-mask softmax in fp64)
# --------------------------------------------------------------------------


def _softmax_rows(s: np.ndarray) -> np.ndarray:
    mx = s.max(axis=1, keepdims=True)
    p = np.exp(s - mx)
    return p / p.sum(axis=1, keepdims=True)


def _workers(workers: Optional[int]) -> int:
    """Worker threads for the per-head loop: the host cores this process may
    use (at most 16), or ``workers`` when given."""
    if workers:
        return max(1, int(workers))
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover - non-Linux hosts
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _for_each(fn, items, workers: int) -> None:
    """Run ``fn(i)`` for every item, on ``workers`` threads with BLAS held to
    one thread each (numpy's element-wise passes release the interpreter
    lock, so heads run side by side; each head's arithmetic is unchanged)."""
    items = list(items)
    if workers <= 1 or len(items) <= 1:
        for i in items:
            fn(i)
        return
    from threadpoolctl import threadpool_limits

    with threadpool_limits(limits=1, user_api="blas"):
        with _cf.ThreadPoolExecutor(min(workers, len(items))) as ex:
            for f in [ex.submit(fn, i) for i in items]:
                f.result()


def attention(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    cu_seqlens: Sequence[int],
    item_id: np.ndarray,
    *,
    scale: Optional[float] = None,
    rows: Optional[np.ndarray] = None,
    row_block: int = 256,
    workers: Optional[int] = None,
) -> np.ndarray:
    """MIS attention output in fp64.

    ``q`` is ``[T, Hq, D]``, ``k``/``v`` are ``[T, Hkv, D]`` (bf16 bits or
    floats). Returns ``[T, Hq, D]``, or ``[len(rows), Hq, D]`` for the packed
    query indices in ``rows`` when given. Every output row is the full softmax
    over all keys of its request with the Eq. 4 mask added. Heads are
    independent and run on ``workers`` threads (default: the host's cores, at
    most 16).
    """
    T, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    nw = _workers(workers)
    want = np.arange(T) if rows is None else np.asarray(rows, dtype=np.int64)
    out = np.zeros((want.shape[0], hq, d))
    req_of = np.searchsorted(np.asarray(cu_seqlens[1:]), want, side="right")
    for r in np.unique(req_of):
        a, b = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        sel = np.nonzero(req_of == r)[0]
        local = want[sel] - a
        ids = item_id[a:b]
        kf, vf = as_f64(k[a:b]), as_f64(v[a:b])
        for c0 in range(0, local.shape[0], row_block):
            lrows = local[c0 : c0 + row_block]
            dst = sel[c0 : c0 + row_block]
            m = mask_rows(ids, lrows)
            qf = as_f64(q[a + lrows])

            def head(h, qf=qf, m=m, dst=dst):
                g = (h * hkv) // hq
                s = scale * (qf[:, h, :] @ kf[:, g, :].T) + m
                out[dst, h, :] = _softmax_rows(s) @ vf[:, g, :]

            _for_each(head, range(hq), nw)
    return out


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, scale: Optional[float] = None):
    """Ordinary causal attention of one sequence (the single-item execution), fp64."""
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    T, hq, d = qf.shape
    hkv = kf.shape[1]
    if scale is None or scale <= 0:
        scale = 1.0 / math.sqrt(d)
    m = np.where(np.arange(T)[None, :] <= np.arange(T)[:, None], 0.0, NEG_INF)
    out = np.zeros((T, hq, d))
    for h in range(hq):
        g = (h * hkv) // hq
        out[:, h, :] = _softmax_rows(scale * (qf[:, h, :] @ kf[:, g, :].T) + m) @ vf[:, g, :]
    return out


def sis_attention(q, k, v, cu_seqlens, prefix_lens, cu_items, item_starts, *, scale=None):
    """Single-item scoring: every item's rows from causal attention over [q; c_i] alone.

    Returns ``[T, Hq, D]`` with the item rows filled (prefix rows come from
    causal attention over the prefix alone).
    """
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    out = np.zeros((qf.shape[0],) + qf.shape[1:])
    for r in range(len(prefix_lens)):
        base, end = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        lq = int(prefix_lens[r])
        pre = np.arange(base, base + lq)
        if lq:
            out[pre] = causal_attention(qf[pre], kf[pre], vf[pre], scale=scale)
        for i in range(int(cu_items[r]), int(cu_items[r + 1])):
            s0 = base + int(item_starts[i])
            s1 = base + (int(item_starts[i + 1]) if i + 1 < int(cu_items[r + 1]) else end - base)
            idx = np.concatenate([pre, np.arange(s0, s1)])
            o = causal_attention(qf[idx], kf[idx], vf[idx], scale=scale)
            out[s0:s1] = o[lq:]
    return out


# --------------------------------------------------------------------------
# rotary position embedding at the reused position ids
# --------------------------------------------------------------------------


def rope(x, pos, theta: float) -> np.ndarray:
    """Rotary embedding of ``x`` ``[T, H, D]`` at positions ``pos`` ``[T]``, fp64.

    Dims i and i + D/2 (i < D/2) are rotated by pos * theta^(-2i/D):
    (a, b) -> (a cos - b sin, b cos + a sin).
    """
    xf = as_f64(x)
    d = xf.shape[-1]
    half = d // 2
    inv = float(theta) ** (-2.0 * np.arange(half, dtype=np.float64) / d)
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a, b = xf[..., :half], xf[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def sis_rope_attention(q, k, v, cu_seqlens, prefix_lens, cu_items, item_starts, theta: float, *,
                       scale=None):
    """Single-item scoring with rotary embedding: every [q; c_i] alone, rotated
    at its own ordinary positions 0 .. Lq + S_i - 1, under a causal mask.

    ``q``/``k`` are the un-rotated inputs. Returns ``[T, Hq, D]`` (prefix rows
    from the prefix alone at positions 0 .. Lq - 1).
    """
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    out = np.zeros((qf.shape[0],) + qf.shape[1:])
    for r in range(len(prefix_lens)):
        base, end = int(cu_seqlens[r]), int(cu_seqlens[r + 1])
        lq = int(prefix_lens[r])
        pre = np.arange(base, base + lq)
        if lq:
            p = np.arange(lq)
            out[pre] = causal_attention(rope(qf[pre], p, theta), rope(kf[pre], p, theta), vf[pre], scale=scale)
        for i in range(int(cu_items[r]), int(cu_items[r + 1])):
            s0 = base + int(item_starts[i])
            s1 = base + (int(item_starts[i + 1]) if i + 1 < int(cu_items[r + 1]) else end - base)
            idx = np.concatenate([pre, np.arange(s0, s1)])
            p = np.arange(len(idx))
            o = causal_attention(rope(qf[idx], p, theta), rope(kf[idx], p, theta), vf[idx], scale=scale)
            out[s0:s1] = o[lq:]
    return out


# --------------------------------------------------------------------------
# label scores (From Generation to Scoring, §3.3 Eq. 2; JEV post's Score API and full-vocab normalisation)
# --------------------------------------------------------------------------


def logits(hidden_rows: np.ndarray, lm_head: np.ndarray, vocab_chunk: int = 16384) -> np.ndarray:
    """Next-token logits ``[N, V]`` = hidden_rows @ lm_head^T in fp64."""
    h = as_f64(hidden_rows)
    V = lm_head.shape[0]
    z = np.empty((h.shape[0], V))
    for v0 in range(0, V, vocab_chunk):
        z[:, v0 : v0 + vocab_chunk] = h @ as_f64(lm_head[v0 : v0 + vocab_chunk]).T
    return z


def label_scores(
    hidden: np.ndarray,
    readout_pos: np.ndarray,
    lm_head: np.ndarray,
    label_ids: Sequence[int],
    *,
    apply_softmax: bool = False,
) -> np.ndarray:
    """One label-score row per item, columns in ``label_ids`` order, fp64.

    The hidden row at each item's readout position is projected onto the
    whole vocabulary. Without ``apply_softmax`` the result is the full-vocab
    log-softmax at the label ids; with it, a softmax over the K label logits.
    """
    rows = np.asarray(hidden)[np.asarray(readout_pos, dtype=np.int64)]
    z = logits(rows, lm_head)
    lab = np.asarray(label_ids, dtype=np.int64)
    zl = z[:, lab]
    if apply_softmax:
        mx = zl.max(axis=1, keepdims=True)
        e = np.exp(zl - mx)
        return e / e.sum(axis=1, keepdims=True)
    mx = z.max(axis=1, keepdims=True)
    lse = mx[:, 0] + np.log(np.exp(z - mx).sum(axis=1))
    return zl - lse[:, None]


def sis_scores(q, k, v, prefix_len: int, item_lens: Sequence[int], lm_head, label_ids, *,
               apply_softmax: bool = False, scale=None) -> np.ndarray:
    """Chained single-item scoring of one request (hidden := attention output, ``Hq*D == H``).

    Each [q; c_i] runs alone with a causal mask; the output row of its last
    token, flattened over heads, is scored against the LM head.
    """
    qf, kf, vf = as_f64(q), as_f64(k), as_f64(v)
    pre = np.arange(prefix_len)
    out = []
    off = prefix_len
    for s in item_lens:
        idx = np.concatenate([pre, np.arange(off, off + int(s))])
        o = causal_attention(qf[idx], kf[idx], vf[idx], scale=scale)
        h_last = o[-1].reshape(1, -1)
        out.append(label_scores(h_last, np.array([0]), lm_head, label_ids,
                                apply_softmax=apply_softmax)[0])
        off += int(s)
    return np.asarray(out)
