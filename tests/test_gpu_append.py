"""Item rows against a cached prefix (mis_attention_append) vs the oracle.

Item rows must equal the full MIS attention (oracle; bit-identical to
mis_attention_prefill's item rows); prefix rows are either left as they were
(checked with a NaN sentinel) or hold the full attention's value.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_ATTN, TOL_F32, build, dev, host, nan_like, say, segments_oracle

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["auto", "pipe", "pipe32", "classic"])
def attention_kernel(request):
    """Each bf16 attention kernel, forced, and the one chosen by shape."""
    mis.set_kernel_choice(attention=request.param)
    yield request.param
    mis.set_kernel_choice()


def _item_mask(wl):
    so = segments_oracle(wl)
    return so["item_id"] >= 0, so


def _append(wl, q, k, v):
    seg = build(wl)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o = nan_like(qd)
    mis.mis_attention_append(seg, qd, kd, vd, o)
    torch.cuda.synchronize()
    return seg, qd, kd, vd, o


@pytest.mark.parametrize("dtype,d,tol", [("bf16", 128, TOL_BF16_ATTN), ("f32", 64, TOL_F32)])
def test_append_item_rows_match_and_prefix_rows_are_kept(dtype, d, tol):
    wl = workloads.from_lengths(f"append-{dtype}", [300, 0, 150, 70], [[9, 40, 1, 65], [5, 3], [], [12] * 5],
                                hq=8, hkv=4, d=d, dtype=dtype, seed=13)
    say(f"[append] {wl.name} T={wl.total_tokens}")
    q, k, v = workloads.qkv(wl)
    _, _, _, _, o = _append(wl, q, k, v)
    got = oracle.as_f64(host(o))
    items, so = _item_mask(wl)
    ref = oracle.attention(q, k, v, wl.cu_seqlens, so["item_id"])
    assert np.abs(got[items] - ref[items]).max() <= tol
    pre = ~items
    kept = np.isnan(got[pre]).all(axis=(1, 2))
    assert np.abs(got[pre][~kept] - ref[pre][~kept]).max(initial=0.0) <= tol
    # prefix rows of query tiles (64 rows) that hold prefix rows only are kept
    for r in range(wl.num_requests):
        base, lq = int(wl.cu_seqlens[r]), int(wl.prefix_lens[r])
        full = (lq // 64) * 64
        assert np.isnan(got[base:base + full]).all(), f"request {r}: prefix-only tiles were rewritten"
    if dtype == "f32":
        assert kept.all()  # the fp32 path skips every prefix row


def test_append_equals_prefill_item_rows_bit_for_bit_single_request_workload():
    wl = workloads.config(2)
    say(f"[append] {wl.name}")
    q, k, v = workloads.qkv(wl)
    seg, qd, kd, vd, o = _append(wl, q, k, v)
    full = host(mis.mis_attention_prefill(seg, qd, kd, vd, o=nan_like(qd)))
    items, _ = _item_mask(wl)
    assert np.array_equal(host(o)[items], full[items])


def test_append_equals_prefill_item_rows_bit_for_bit_long_visit_lists():
    # a 4200-token prefix: item tiles visit 67 key tiles, the first partly
    # visible one (the prefix's last) past the first 64
    wl = workloads.from_lengths("append-long", [4200, 130], [[5, 9, 40], [7, 7]], hq=8, hkv=2, d=128, seed=23)
    say(f"[append] {wl.name} T={wl.total_tokens}")
    q, k, v = workloads.qkv(wl)
    seg, qd, kd, vd, o = _append(wl, q, k, v)
    full = host(mis.mis_attention_prefill(seg, qd, kd, vd, o=nan_like(qd)))
    items, _ = _item_mask(wl)
    assert np.array_equal(host(o)[items], full[items])
