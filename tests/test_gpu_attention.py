"""GPU MIS attention vs the fp64 oracle (element by element), plus SIS, order and determinism checks.

Every output starts as NaN, so a query row that no kernel writes fails the
finiteness check over the whole output. Small shapes, the single-request and
the profile-labeling workloads are compared on every output element; the
ragged serving batch and the long-prefix workload on the first and last row
of every 64-row query tile (every head, every dim; the ragged batch also on a
random row of every tile), in the launch configuration the benchmark times.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import (TOL_BF16_ATTN, TOL_F32, attention, build, cached, host, say, segments_oracle,
                        tile_rows)

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["auto", "pipe", "pipe2", "pipe32", "classic"])
def attention_kernel(request):
    """Run every case with the bf16 kernel chosen by shape, and forced to each
    of the three kernels (the pipelined loop with 64 or with 32 query rows per
    wave, or the plain loop with two waves per SIMD); the fp32 cases do not
    depend on it."""
    mis.set_kernel_choice(attention=request.param)
    yield request.param
    mis.set_kernel_choice()


def _err(got, ref):
    return float(np.abs(oracle.as_f64(got) - ref).max())


def _inputs(wl, scale_q=1.0):
    if wl.name in ("profile-labeling-bf16", "ragged-serving-bf16", "long-prefix-bf16"):
        return cached(("qkv", wl.name, scale_q), lambda: workloads.qkv(wl, scale_q=scale_q))
    return workloads.qkv(wl, scale_q=scale_q)


def _run(wl, scale_q=1.0):
    q, k, v = _inputs(wl, scale_q)
    seg = build(wl)
    o = host(attention(wl, seg, q, k, v))
    return q, k, v, o


def _full_check(wl, scale_q=1.0, tol=None):
    tol = tol or (TOL_F32 if wl.dtype == "f32" else TOL_BF16_ATTN)
    say(f"[attention full] {wl.name} T={wl.total_tokens} hq={wl.hq} hkv={wl.hkv}")
    q, k, v, o = _run(wl, scale_q)
    ref = cached(("attn-full", wl.name, wl.seed, scale_q, wl.total_tokens, wl.hq, wl.hkv),
                 lambda: oracle.attention(q, k, v, wl.cu_seqlens, segments_oracle(wl)["item_id"]))
    e = _err(o, ref)
    say(f"  max abs err {e:.3e}")
    assert np.isfinite(oracle.as_f64(o)).all()
    assert e <= tol
    return q, k, v, o


def test_f32_tiny_config():
    _full_check(workloads.config(1))


def test_f32_d128_and_gqa():
    wl = workloads.from_lengths("f32gqa", [37, 0], [[5, 1, 12], [3, 3]], dtype="f32", hq=6, hkv=2,
                                d=128, seed=7)
    _full_check(wl)


@pytest.mark.parametrize("shape", [
    ([130], [[9, 1, 33, 64, 2]], 8, 4),
    ([0, 77, 200], [[40, 1, 1], [5, 70], [3] * 20], 8, 2),
    ([65], [[]], 4, 2),  # T = 65: last query/key tile holds one token
    ([129, 1], [[1, 1, 1], []], 16, 8),
    ([300], [[17] * 12], 4, 4),  # G = 1 (MHA) uses the one-head workgroup
    ([64, 63], [[64], [1, 1]], 6, 2),  # odd group size (3)
    # 67 visits per item tile: the first partly visible tile (the prefix's
    # last) is visit 65, past the 64 a wave's lanes cover in one pass
    ([4200], [[5, 9, 40]], 8, 2),
])
def test_bf16_small_shapes_all_elements(shape):
    p, it, hq, hkv = shape
    wl = workloads.from_lengths("small", p, it, hq=hq, hkv=hkv, d=128, seed=len(p) * 31 + hq)
    _full_check(wl)


def test_bf16_peaky_softmax():
    # Q x 4 sharpens the softmax: exercises online-max raising and rescaling
    wl = workloads.from_lengths("peaky", [700], [[20] * 30], hq=8, hkv=4, d=128, seed=9)
    _full_check(wl, scale_q=4.0)


def test_bf16_single_request_config_full():
    _full_check(workloads.config(2))


def _tile_check(k_cfg, extra_per_tile):
    wl = workloads.config(k_cfg)
    say(f"[attention per tile] {wl.name} T={wl.total_tokens}")
    q, k, v, o = _run(wl)
    rows = tile_rows(wl, extra_per_tile=extra_per_tile, seed=k_cfg)

    def ref_rows():
        say(f"  oracle on {len(rows)} rows x {wl.hq} heads")
        return oracle.attention(q, k, v, wl.cu_seqlens, segments_oracle(wl)["item_id"], rows=rows)

    ref = cached(("attn-tiles", wl.name), ref_rows)
    e = _err(o[rows], ref)
    say(f"  {len(rows)} rows, max abs err {e:.3e}")
    assert np.isfinite(oracle.as_f64(o)).all()
    assert e <= TOL_BF16_ATTN


def test_bf16_profile_labeling_config_full():
    _full_check(workloads.config(3))


def test_bf16_ragged_serving_config_every_tile():
    _tile_check(4, 1)


def test_bf16_long_prefix_config_every_tile():
    _tile_check(5, 0)


def test_mis_rows_equal_single_item_scoring():
    # every item of a small batch, against [q; c_i] run alone under a causal mask
    wl = workloads.from_lengths("sis", [96, 40], [[7, 30, 1, 12], [25, 2]], hq=8, hkv=4, d=128,
                                seed=12)
    q, k, v, o = _run(wl)
    sis = oracle.sis_attention(q, k, v, wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    assert _err(o, sis) <= TOL_BF16_ATTN


def test_f32_tiny_config_equals_single_item_scoring():
    wl = workloads.config(1)
    q, k, v, o = _run(wl)
    sis = oracle.sis_attention(q, k, v, wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)
    assert _err(o, sis) <= TOL_F32


def test_item_order_invariance():
    lens = [9, 33, 1, 17, 64, 5]
    perm = [3, 0, 5, 1, 4, 2]
    wl = workloads.from_lengths("order", [150], [lens], hq=8, hkv=4, d=128, seed=13)
    q, k, v, o = _run(wl)
    wl2 = workloads.from_lengths("order2", [150], [[lens[p] for p in perm]], hq=8, hkv=4, d=128)
    idx = list(range(150))
    for p in perm:
        s0 = int(wl.item_starts[p])
        idx += list(range(s0, s0 + lens[p]))
    idx = np.asarray(idx)
    seg2 = build(wl2)
    o2 = host(attention(wl2, seg2, q[idx], k[idx], v[idx]))
    assert _err(o2, oracle.as_f64(o[idx])) <= TOL_BF16_ATTN


def test_repeat_runs_are_bit_identical():
    # both outputs start as NaN, so neither can inherit the other's values
    wl = workloads.config(2)
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    a = host(attention(wl, seg, q, k, v))
    b = host(attention(wl, seg, q, k, v))
    assert np.isfinite(oracle.as_f64(a)).all()
    assert np.array_equal(a, b)


def test_explicit_softmax_scale():
    wl = workloads.from_lengths("scale", [80], [[10, 20]], hq=8, hkv=4, d=128, seed=14)
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    o = host(attention(wl, seg, q, k, v, scale=0.05))
    ref = oracle.attention(q, k, v, wl.cu_seqlens, segments_oracle(wl)["item_id"], scale=0.05)
    assert _err(o, ref) <= TOL_BF16_ATTN
