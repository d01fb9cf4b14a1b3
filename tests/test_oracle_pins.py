"""Pins of the fp64 oracle to facts outside itself (CPU only).

* Figure 2 of "From Generation to Scoring" (§4.1), transcribed by hand into
  ``tests/golden/fig2_mis_mask.txt``: mask, reused position ids, readout rows,
  and tile classes worked out by hand from that mask.
* torch's ``scaled_dot_product_attention`` in float64 on the CPU (a second,
  independent attention routine): ordinary causal attention for N=1, for
  Lq=0, and for every [q; c_i] run alone (single-item scoring, which MIS must
  reproduce: §4.1 and Table 1's release check).
* Invariance of item scores to item order (§4.1 and §6.2).
* Closed form of the number of visible (query, key) pairs, from §4.3's
  statement that the query attends to itself once and each item to the
  query plus its own causal prefix.
* Label scores: pure-Python brute force on a tiny vocabulary, scipy's
  logsumexp, total probability one over the whole vocabulary, and Eq. 2
  (two-label renormalisation is the logistic of the logit difference).

The planted-mistake tests at the end break the oracle on purpose (on the
CPU only) and check that some pin fails for each mistake.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F
from hypothesis import given, settings, strategies as st

import oracle
import oracle.mis as om
import workloads
from helpers import read_golden

torch.set_num_threads(4)


# ---------------------------------------------------------------- helpers


def _wl(prefix_lens, item_lens, hq=4, hkv=2, d=16, seed=0, **kw):
    return workloads.from_lengths("t", prefix_lens, item_lens, seed=seed, dtype="f32",
                                  hq=hq, hkv=hkv, d=d, **kw)


def _segs(wl):
    return oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)


def _sdpa(q, k, v, *, causal=False, mask=None, scale=None):
    """torch SDPA in float64; q [T,Hq,D], k/v [T,Hkv,D]; contiguous GQA groups."""
    qt = torch.from_numpy(oracle.as_f64(q)).permute(1, 0, 2)[None]
    kt = torch.from_numpy(oracle.as_f64(k)).permute(1, 0, 2)[None]
    vt = torch.from_numpy(oracle.as_f64(v)).permute(1, 0, 2)[None]
    g = qt.shape[1] // kt.shape[1]
    kt = kt.repeat_interleave(g, dim=1)
    vt = vt.repeat_interleave(g, dim=1)
    am = None if mask is None else torch.from_numpy(mask)
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=am, is_causal=causal, scale=scale)
    return o[0].permute(1, 0, 2).numpy()


def _sis_by_sdpa(wl, q, k, v):
    """Every item's rows from SDPA causal attention over [q; c_i]; prefix rows over q alone."""
    out = np.zeros(q.shape, dtype=np.float64)
    for r in range(wl.num_requests):
        base = int(wl.cu_seqlens[r])
        lq = int(wl.prefix_lens[r])
        pre = np.arange(base, base + lq)
        if lq:
            out[pre] = _sdpa(q[pre], k[pre], v[pre], causal=True)
        lens = wl.item_lengths()
        for i in range(int(wl.cu_items[r]), int(wl.cu_items[r + 1])):
            s0 = base + int(wl.item_starts[i])
            idx = np.concatenate([pre, np.arange(s0, s0 + int(lens[i]))])
            out[s0 : s0 + int(lens[i])] = _sdpa(q[idx], k[idx], v[idx], causal=True)[lq:]
    return out


def _closed_form_pairs(lq, item_lens):
    return lq * (lq + 1) // 2 + sum(s * lq + s * (s + 1) // 2 for s in item_lens)


def _mis(wl, q, k, v, **kw):
    return oracle.attention(q, k, v, wl.cu_seqlens, _segs(wl)["item_id"], **kw)


# ------------------------------------------------------------ Figure 2 pins


def check_fig2() -> bool:
    g = read_golden("fig2_mis_mask.txt")
    wl = _wl(g["prefix_len"], [g["item_lens"]])
    seg = _segs(wl)
    ok = list(seg["pos_id"]) == g["pos_id"]
    ok &= list(seg["readout_pos"]) == g["readout_pos"]
    vis = (oracle.mis_mask(seg["item_id"]) == 0.0).astype(int)
    ok &= vis.tolist() == g["mask"]
    for (bm, bn), grid in g["tiles"].items():
        cls, cu = oracle.tile_classes(wl.cu_seqlens, seg["item_id"], bm, bn)
        ok &= cls.reshape(len(grid), len(grid[0])).tolist() == grid
    return bool(ok)


def test_fig2_mask_positions_readout_and_tiles():
    assert check_fig2()


def test_fig2_item_ids():
    g = read_golden("fig2_mis_mask.txt")
    seg = _segs(_wl(g["prefix_len"], [g["item_lens"]]))
    assert seg["item_id"].tolist() == [-1, -1, -1, -1, 0, 0, 1, 1, 2, 2]


# ------------------------------------------------------- attention pins


def check_sis(wl, q, k, v) -> float:
    return float(np.abs(_mis(wl, q, k, v) - _sis_by_sdpa(wl, q, k, v)).max())


def check_sdpa_same_mask(wl, q, k, v) -> float:
    seg = _segs(wl)
    err = 0.0
    mis = _mis(wl, q, k, v)
    for r in range(wl.num_requests):
        a, b = int(wl.cu_seqlens[r]), int(wl.cu_seqlens[r + 1])
        allowed = oracle.mis_mask(seg["item_id"][a:b]) == 0.0
        ref = _sdpa(q[a:b], k[a:b], v[a:b], mask=allowed)
        err = max(err, float(np.abs(mis[a:b] - ref).max()))
    return err


def _qkv(wl, scale_q=1.0):
    return workloads.qkv(wl, scale_q=scale_q)


def test_single_item_is_plain_causal():
    wl = _wl([13], [[7]], seed=3)
    q, k, v = _qkv(wl)
    assert np.abs(_mis(wl, q, k, v) - _sdpa(q, k, v, causal=True)).max() < 1e-12


def test_no_prefix_gives_independent_causal_items():
    wl = _wl([0], [[5, 1, 9, 3]], seed=4)
    q, k, v = _qkv(wl)
    out = _mis(wl, q, k, v)
    for s0, n in zip(wl.item_starts, wl.item_lengths()):
        sl = slice(int(s0), int(s0 + n))
        assert np.abs(out[sl] - _sdpa(q[sl], k[sl], v[sl], causal=True)).max() < 1e-12


def test_no_items_is_plain_causal():
    wl = _wl([21], [[]], seed=5)
    q, k, v = _qkv(wl)
    assert np.abs(_mis(wl, q, k, v) - _sdpa(q, k, v, causal=True)).max() < 1e-12


def test_mis_equals_single_item_scoring_small():
    wl = _wl([11, 0, 6], [[3, 1, 5], [4, 2], [1]], hq=6, hkv=3, seed=6)
    q, k, v = _qkv(wl, scale_q=3.0)
    assert check_sis(wl, q, k, v) < 1e-12


def test_matches_sdpa_under_same_mask_with_gqa():
    wl = _wl([9, 5], [[4, 4], [2, 7, 1]], hq=8, hkv=2, seed=7)
    q, k, v = _qkv(wl)
    assert check_sdpa_same_mask(wl, q, k, v) < 1e-12


def test_explicit_scale_is_used():
    wl = _wl([6], [[3, 2]], seed=8)
    q, k, v = _qkv(wl)
    seg = _segs(wl)
    out = oracle.attention(q, k, v, wl.cu_seqlens, seg["item_id"], scale=0.37)
    ref = _sdpa(q, k, v, mask=oracle.mis_mask(seg["item_id"]) == 0.0, scale=0.37)
    assert np.abs(out - ref).max() < 1e-12


def test_first_row_of_each_request_is_its_value_row():
    wl = _wl([4, 0], [[3], [2, 2]], hq=4, hkv=2, seed=9)
    q, k, v = _qkv(wl)
    out = _mis(wl, q, k, v)
    for r in range(wl.num_requests):
        t = int(wl.cu_seqlens[r])
        for h in range(4):
            assert np.array_equal(out[t, h], oracle.as_f64(v[t, h // 2]))


def test_item_order_does_not_change_item_rows():
    lens = [4, 1, 6, 3]
    perm = [2, 0, 3, 1]
    wl = _wl([10], [lens], seed=10)
    q, k, v = _qkv(wl)
    out = _mis(wl, q, k, v)
    wl2 = _wl([10], [[lens[p] for p in perm]], seed=10)
    idx = list(range(10))
    for p in perm:
        s0 = int(wl.item_starts[p])
        idx += list(range(s0, s0 + lens[p]))
    idx = np.asarray(idx)
    out2 = _mis(wl2, q[idx], k[idx], v[idx])
    assert np.abs(out2 - out[idx]).max() < 1e-12


def test_sampled_rows_equal_full_rows():
    wl = _wl([17, 5], [[3, 8], [6]], seed=11)
    q, k, v = _qkv(wl)
    full = _mis(wl, q, k, v)
    rows = np.array([0, 5, 16, 17, 27, 28, 29, 38])
    part = _mis(wl, q, k, v, rows=rows)
    assert np.array_equal(part, full[rows])


@settings(max_examples=25, deadline=None)
@given(st.data())
def test_property_mis_equals_sis(data):
    nreq = data.draw(st.integers(1, 3))
    prefix, items = [], []
    for _ in range(nreq):
        lq = data.draw(st.integers(0, 40))
        n = data.draw(st.integers(0 if lq else 1, 8))
        prefix.append(lq)
        items.append(data.draw(st.lists(st.integers(1, 12), min_size=n, max_size=n)))
    g = data.draw(st.sampled_from([1, 2, 4]))
    wl = _wl(prefix, items, hq=2 * g, hkv=2, d=8, seed=data.draw(st.integers(0, 1000)))
    q, k, v = _qkv(wl)
    assert check_sis(wl, q, k, v) < 1e-12


# ----------------------------------------------------- segment / tile pins


@settings(max_examples=40, deadline=None)
@given(st.integers(0, 60), st.lists(st.integers(1, 15), min_size=0, max_size=10))
def test_visible_pairs_closed_form(lq, lens):
    if lq == 0 and not lens:
        lens = [1]
    wl = _wl([lq], [lens])
    assert oracle.visible_pairs(_segs(wl)["item_id"]) == _closed_form_pairs(lq, lens)


def test_positions_restart_per_item_and_request():
    wl = _wl([3, 2], [[2, 3], [1, 2]])
    seg = _segs(wl)
    assert seg["pos_id"].tolist() == [0, 1, 2, 3, 4, 3, 4, 5, 0, 1, 2, 2, 3]
    assert seg["item_id"].tolist() == [-1, -1, -1, 0, 0, 1, 1, 1, -1, -1, 2, 3, 3]
    assert seg["readout_pos"].tolist() == [4, 7, 10, 12]
    # largest position id is Lq + max item length - 1 (§4.4 request sizing)
    assert seg["pos_id"][:8].max() == 3 + 3 - 1


@settings(max_examples=30, deadline=None)
@given(st.integers(0, 50), st.lists(st.integers(1, 13), min_size=0, max_size=8),
       st.sampled_from([1, 2, 3, 4, 8, 16]), st.sampled_from([1, 2, 4, 5, 16]))
def test_tile_classes_agree_with_visible_counts(lq, lens, bm, bn):
    if lq == 0 and not lens:
        lens = [2]
    wl = _wl([lq], [lens])
    ids = _segs(wl)["item_id"]
    cls, cu = oracle.tile_classes(wl.cu_seqlens, ids, bm, bn)
    vis = oracle.mis_mask(ids) == 0.0
    T = ids.shape[0]
    nkt = -(-T // bn)
    assert cu.tolist() == [0, -(-T // bm) * nkt]
    for t, c in enumerate(cls):
        qt, kt = divmod(t, nkt)
        blk = vis[qt * bm : (qt + 1) * bm, kt * bn : (kt + 1) * bn]
        # a tile holding the diagonal always has a visible cell
        if qt * bm < (kt + 1) * bn and kt * bn < (qt + 1) * bm and kt * bn < T:
            assert c != 0
        assert c == (0 if not blk.any() else (2 if blk.all() else 1))
    if bm == 1 and bn == 1:  # 1x1 tiles are the mask itself
        assert ((cls == 2).reshape(T, T) == vis).all()


# -------------------------------------------------------- label-score pins


def _brute_logprobs(hrows, W, labels):
    out = []
    for h in hrows:
        z = [math.fsum(float(h[j]) * float(W[v, j]) for j in range(len(h))) for v in range(W.shape[0])]
        m = max(z)
        lse = m + math.log(math.fsum(math.exp(x - m) for x in z))
        out.append([z[l] - lse for l in labels])
    return np.array(out)


def check_label_scores_brute() -> float:
    rng = np.random.default_rng(0)
    T, H, V = 7, 8, 50
    hidden = np.full((T, H), np.nan)
    readout = np.array([2, 4, 6])
    hidden[readout] = rng.standard_normal((3, H))
    W = rng.standard_normal((V, H))
    labels = [7, 3, 7, 49]
    got = oracle.label_scores(hidden, readout, W, labels)
    return float(np.abs(got - _brute_logprobs(hidden[readout], W, labels)).max())


def test_label_scores_match_brute_force_and_skip_other_rows():
    assert check_label_scores_brute() < 1e-12


def test_label_scores_match_scipy_logsumexp():
    rng = np.random.default_rng(1)
    N, H, V = 5, 32, 5000
    h = rng.standard_normal((N, H))
    W = 0.02 * rng.standard_normal((V, H))
    labels = rng.choice(V, 3, replace=False)
    got = oracle.label_scores(h, np.arange(N), W, labels)
    z = h @ W.T
    ref = z[:, labels] - scipy.special.logsumexp(z, axis=1)[:, None]
    assert np.abs(got - ref).max() < 1e-12


def test_whole_vocab_probabilities_sum_to_one():
    rng = np.random.default_rng(2)
    N, H, V = 4, 16, 300
    h = 3.0 * rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    lp = oracle.label_scores(h, np.arange(N), W, np.arange(V))
    assert (lp <= 0).all()
    assert np.abs(np.exp(lp).sum(axis=1) - 1.0).max() < 1e-12


def test_two_label_softmax_is_eq2():
    rng = np.random.default_rng(3)
    N, H, V = 6, 16, 100
    h = rng.standard_normal((N, H))
    W = rng.standard_normal((V, H))
    yes, no = 17, 42
    p = oracle.label_scores(h, np.arange(N), W, [yes, no], apply_softmax=True)
    z = h @ W.T
    assert np.abs(p[:, 0] - scipy.special.expit(z[:, yes] - z[:, no])).max() < 1e-12
    assert np.abs(p.sum(axis=1) - 1.0).max() < 1e-12
    # renormalised label scores do not depend on the rest of the vocabulary
    W2 = W.copy()
    W2[[i for i in range(V) if i not in (yes, no)]] *= 5.0
    p2 = oracle.label_scores(h, np.arange(N), W2, [yes, no], apply_softmax=True)
    assert np.abs(p - p2).max() < 1e-12


def test_chained_mis_scores_equal_single_item_scores():
    # hidden := attention output flattened over heads (Hq*D == H), read at each item's last token
    wl = _wl([12], [[4, 6, 2]], hq=4, hkv=4, d=8, seed=12)
    q, k, v = _qkv(wl)
    rng = np.random.default_rng(4)
    W = rng.standard_normal((60, 32))
    labels = [5, 9]
    seg = _segs(wl)
    hid = _mis(wl, q, k, v).reshape(wl.total_tokens, -1)
    mis = oracle.label_scores(hid, seg["readout_pos"], W, labels)
    sis = oracle.sis_scores(q, k, v, 12, [4, 6, 2], W, labels)
    # independent route: SDPA for each [q; c_i], scipy for the normalisation
    ref = []
    for s0, n in zip(wl.item_starts, wl.item_lengths()):
        idx = np.concatenate([np.arange(12), np.arange(s0, s0 + n)])
        h_last = _sdpa(q[idx], k[idx], v[idx], causal=True)[-1].reshape(-1)
        z = W @ h_last
        ref.append(z[labels] - scipy.special.logsumexp(z))
    assert np.abs(mis - np.array(ref)).max() < 1e-12
    assert np.abs(sis - np.array(ref)).max() < 1e-12


# ------------------------------------------------------ planted mistakes


def _bad_mask_no_item_causality(ids, rows):
    ids = np.asarray(ids)
    rows = np.asarray(rows)
    T = ids.shape[0]
    causal = np.arange(T)[None, :] <= rows[:, None]
    kq = (ids == -1)[None, :]
    same = (ids[rows][:, None] == ids[None, :]) & (ids[rows][:, None] >= 0)
    m = np.full((rows.shape[0], T), -np.inf)
    m[(causal & kq) | same] = 0.0  # items see their own future tokens
    return m


def _bad_mask_cross_item(ids, rows):
    ids = np.asarray(ids)
    rows = np.asarray(rows)
    T = ids.shape[0]
    causal = np.arange(T)[None, :] <= rows[:, None]
    m = np.full((rows.shape[0], T), -np.inf)
    m[causal] = 0.0  # plain causal: items see earlier items
    return m


def _bad_mask_transposed(ids, rows):
    ids = np.asarray(ids)
    T = ids.shape[0]
    allr = np.arange(T)
    good = _ORIG_MASK_ROWS(ids, allr)
    return good.T[np.asarray(rows)]


_ORIG_MASK_ROWS = om.mask_rows


def _fixture_inputs():
    wl = _wl([6, 3], [[3, 2, 4], [2, 1]], hq=4, hkv=2, seed=21)
    q, k, v = _qkv(wl)
    return wl, q, k, v


@pytest.mark.parametrize("bad", [_bad_mask_no_item_causality, _bad_mask_cross_item,
                                 _bad_mask_transposed])
def test_planted_mask_mistakes_are_caught(monkeypatch, bad):
    monkeypatch.setattr(om, "mask_rows", bad)
    wl, q, k, v = _fixture_inputs()
    assert not check_fig2()
    assert check_sis(wl, q, k, v) > 1e-3


def test_planted_gqa_mapping_mistake_is_caught(monkeypatch):
    orig = om.attention

    def bad(q, k, v, *a, **kw):  # query head h reads kv head h % Hkv instead of its group
        hq, hkv = q.shape[1], k.shape[1]
        perm = np.array([(h % hkv) for h in range(hq)])
        qq = np.concatenate([q[:, perm == g] for g in range(hkv)], axis=1)
        order = np.concatenate([np.nonzero(perm == g)[0] for g in range(hkv)])
        o = orig(qq, k, v, *a, **kw)
        out = np.empty_like(o)
        out[:, order] = o
        return out

    monkeypatch.setattr(oracle, "attention", bad)
    wl, q, k, v = _fixture_inputs()
    assert check_sdpa_same_mask(wl, q, k, v) > 1e-3


def test_planted_missing_scale_is_caught(monkeypatch):
    orig = om.attention
    monkeypatch.setattr(oracle, "attention", lambda *a, **kw: orig(*a, **{**kw, "scale": 1.0}))
    wl, q, k, v = _fixture_inputs()
    assert check_sdpa_same_mask(wl, q, k, v) > 1e-3


def test_planted_segment_mistakes_are_caught(monkeypatch):
    orig = om.build_segments

    def readout_at_item_start(*a):
        s = orig(*a)
        s = dict(s)
        s["readout_pos"] = s["readout_pos"] - 1
        return s

    def global_positions(*a):
        s = dict(orig(*a))
        s["pos_id"] = np.arange(s["pos_id"].shape[0])
        return s

    for bad in (readout_at_item_start, global_positions):
        monkeypatch.setattr(oracle, "build_segments", bad)
        assert not check_fig2()
    monkeypatch.setattr(oracle, "build_segments", orig)
    assert check_fig2()


def test_planted_label_normalisation_mistake_is_caught(monkeypatch):
    orig = om.label_scores

    def labels_only_lse(hidden, readout, W, labels, apply_softmax=False):
        z = om.logits(np.asarray(hidden)[readout], W)[:, labels]
        return z - scipy.special.logsumexp(z, axis=1)[:, None]

    monkeypatch.setattr(oracle, "label_scores", labels_only_lse)
    assert check_label_scores_brute() > 1e-3
    monkeypatch.setattr(oracle, "label_scores", orig)
    assert check_label_scores_brute() < 1e-12
