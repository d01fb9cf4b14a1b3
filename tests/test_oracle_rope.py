"""Pins of the oracle's rotary embedding at the reused position ids.

The rotation is pinned by a hand-worked example, by properties the rotary
embedding must have (identity at position 0, norm of every pair kept, scores
depend on the position difference only) and by planted mistakes; the reused
positions are pinned by the MIS = SIS equivalence with rotation applied
(each [q; c_i] alone at ordinary positions 0 .. Lq + S_i - 1).
"""
import math

import numpy as np
import pytest

import oracle
import oracle.mis as om
import workloads


def test_hand_worked_example():
    # D = 4, theta = 100: pair (0, 2) turns by pos * 1, pair (1, 3) by pos * 0.1
    x = np.zeros((1, 1, 4))
    x[0, 0] = [1.0, 0.0, 0.0, 0.0]
    y = oracle.rope(x, [2], 100.0)[0, 0]
    assert np.allclose(y, [math.cos(2.0), 0.0, math.sin(2.0), 0.0], atol=1e-15)
    x[0, 0] = [0.0, 1.0, 0.0, 0.0]
    y = oracle.rope(x, [2], 100.0)[0, 0]
    assert np.allclose(y, [0.0, math.cos(0.2), 0.0, math.sin(0.2)], atol=1e-15)
    x[0, 0] = [0.0, 0.0, 0.0, 1.0]  # second member of the pair turns the other way round
    y = oracle.rope(x, [3], 100.0)[0, 0]
    assert np.allclose(y, [0.0, -math.sin(0.3), 0.0, math.cos(0.3)], atol=1e-15)


def test_position_zero_is_identity_and_pairs_keep_their_norm():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 16))
    pos = np.array([0, 1, 5, 17, 100, 3000, 65000])
    y = oracle.rope(x, pos, 1e4)
    assert np.array_equal(y[0], x[0])
    nx = x[..., :8] ** 2 + x[..., 8:] ** 2
    ny = y[..., :8] ** 2 + y[..., 8:] ** 2
    assert np.allclose(nx, ny, rtol=1e-12)


@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_scores_depend_on_position_difference_only(theta):
    rng = np.random.default_rng(1)
    qv = rng.standard_normal((1, 1, 32))
    kv = rng.standard_normal((1, 1, 32))
    def score(m, n):
        return float(np.sum(oracle.rope(qv, [m], theta) * oracle.rope(kv, [n], theta)))
    for m, n in [(5, 2), (40, 40), (7, 30), (1000, 999)]:
        for shift in (1, 13, 2048):
            assert abs(score(m, n) - score(m + shift, n + shift)) < 1e-9
    assert abs(score(5, 2) - score(6, 2)) > 1e-6  # and it does depend on the difference


def _wl():
    return workloads.from_lengths("rope", [9, 0, 5], [[3, 4, 1], [2, 6], []], hq=4, hkv=2, d=16, seed=3)


def test_mis_with_rope_at_reused_positions_equals_single_item_scoring():
    wl = _wl()
    q, k, v = workloads.qkv(wl)
    seg = oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    theta = 1e4
    qr = oracle.rope(q, seg["pos_id"], theta)
    kr = oracle.rope(k, seg["pos_id"], theta)
    mis = oracle.attention(qr, kr, v, wl.cu_seqlens, seg["item_id"])
    sis = oracle.sis_rope_attention(q, k, v, wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, theta)
    assert np.max(np.abs(mis - sis)) < 1e-12
    # packed positions 0 .. T_r - 1 instead of the reused ones break it
    packed = np.concatenate([np.arange(wl.cu_seqlens[r + 1] - wl.cu_seqlens[r]) for r in range(wl.num_requests)])
    bad = oracle.attention(oracle.rope(q, packed, theta), oracle.rope(k, packed, theta), v, wl.cu_seqlens,
                           seg["item_id"])
    assert np.max(np.abs(bad - sis)) > 1e-3


def _rope_interleaved(x, pos, theta):  # planted: pairs (2i, 2i+1) instead of (i, i + D/2)
    xf = om.as_f64(x)
    d = xf.shape[-1]
    inv = theta ** (-2.0 * np.arange(d // 2) / d)
    ang = np.asarray(pos, float)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    a, b = xf[..., 0::2], xf[..., 1::2]
    out = np.empty_like(xf)
    out[..., 0::2] = a * c - b * s
    out[..., 1::2] = b * c + a * s
    return out


def _rope_wrong_sign(x, pos, theta):  # planted: rotation by -angle
    return om.rope(x, -np.asarray(pos, float), theta)


@pytest.mark.parametrize("bad", [_rope_interleaved, _rope_wrong_sign])
def test_planted_rotation_mistakes_fail_the_hand_example(monkeypatch, bad):
    monkeypatch.setattr(oracle, "rope", bad)
    with pytest.raises(AssertionError):
        test_hand_worked_example()
