"""The profile-labeling benchmark's shape (From Generation to Scoring, §6.1:
queries of median 543 / mean 744 tokens, 200 items of 28 tokens per member),
a small seeded draw of two members, through the C ABI.

MIS attention is checked on every output element and the label log-probs of
every item against the fp64 oracle. The same rows laid out as two requests
of 100 items per member (§6.4's split) and as one request per item
(single-item scoring) must give the same item rows and scores as MIS, within
the bf16 tolerances (tile alignment differs between the layouts).
"""
import numpy as np
import pytest
import torch

import bench
import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_ATTN, TOL_BF16_SCORE, cached, dev, host, nan_like, say, segments_oracle

pytestmark = pytest.mark.gpu


def _case():
    wl = workloads.paper_batch(2, 200, 28, seed=61)
    q, k, v = workloads.qkv(wl)
    so = segments_oracle(wl)
    hid = np.zeros((wl.total_tokens, wl.hidden), dtype=np.uint16)
    hid[so["readout_pos"]] = workloads.readout_values(wl)
    W = workloads.lm_head(wl)
    labels = workloads.label_ids(wl)
    say(f"[paper] T={wl.total_tokens} queries {wl.prefix_lens.tolist()}: oracle")
    ref_o = oracle.attention(q, k, v, wl.cu_seqlens, so["item_id"])
    ref_s = oracle.label_scores(hid, so["readout_pos"], W, labels)
    return wl, dev(q), dev(k), dev(v), dev(hid), dev(W), labels, so, ref_o, ref_s


def _run(wl, requests, qd, kd, vd, hd, Wd, labels):
    rows, cu, pl, ci, st = bench.layout(wl, requests)
    idx = torch.from_numpy(rows).cuda()
    qx, kx, vx, hx = qd[idx], kd[idx], vd[idx], hd[idx]
    bm, bn = mis.mis_attention_tile_shape(mis.MIS_BF16, wl.hq, wl.hkv, wl.d)
    seg = mis.mis_build_segments(cu, pl, ci, st, bm, bn)
    o = nan_like(qx)
    mis.mis_attention_prefill(seg, qx, kx, vx, o=o)
    s = mis.mis_score_labels(seg, hx, Wd, labels)
    torch.cuda.synchronize()
    return rows, oracle.as_f64(host(o)), host(s).astype(np.float64)


def test_paper_shape_mis_against_the_oracle_and_other_layouts():
    wl, qd, kd, vd, hd, Wd, labels, so, ref_o, ref_s = cached(("paper", 61), _case)
    members = range(wl.num_requests)
    rows, o, s = _run(wl, [(r, range(200)) for r in members], qd, kd, vd, hd, Wd, labels)
    assert np.array_equal(rows, np.arange(wl.total_tokens))
    assert np.isfinite(o).all() and np.isfinite(s).all()
    e_o, e_s = float(np.abs(o - ref_o).max()), float(np.abs(s - ref_s).max())
    say(f"  MIS: attention max abs err {e_o:.3e}, label log-probs {e_s:.3e}")
    assert e_o <= TOL_BF16_ATTN and e_s <= TOL_BF16_SCORE

    items = so["item_id"] >= 0
    for name, reqs in (("split 2 x 100", [(r, range(h * 100, (h + 1) * 100)) for r in members for h in (0, 1)]),
                       ("single-item", [(r, [i]) for r in members for i in range(200)])):
        rows_x, o_x, s_x = _run(wl, reqs, qd, kd, vd, hd, Wd, labels)
        assert np.isfinite(o_x).all() and np.isfinite(s_x).all()
        # every item row of the layout against the same row under MIS and the oracle
        item_rows = items[rows_x]
        e_mis = float(np.abs(o_x[item_rows] - o[rows_x[item_rows]]).max())
        e_ref = float(np.abs(o_x[item_rows] - ref_o[rows_x[item_rows]]).max())
        e_sc = float(np.abs(s_x - ref_s).max())  # items keep their global order in both layouts
        say(f"  {name}: item rows vs MIS {e_mis:.3e}, vs oracle {e_ref:.3e}; scores vs oracle {e_sc:.3e}")
        assert e_ref <= TOL_BF16_ATTN and e_mis <= 2 * TOL_BF16_ATTN and e_sc <= TOL_BF16_SCORE
