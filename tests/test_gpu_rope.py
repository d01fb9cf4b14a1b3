"""GPU rotary embedding at the reused position ids vs the oracle.

bf16 results are rounded once to bf16, so the bound is half a bf16 unit in
the last place of the exact value (2^-8 relative) plus the fp32 arithmetic;
fp32 results meet the fp32 bound (1e-4). With the rotation applied, MIS
attention on the GPU must equal the oracle's single-item scoring at ordinary
positions.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_ATTN, TOL_F32, build, dev, host, nan_like, say, segments_oracle

pytestmark = pytest.mark.gpu


def _gpu_rope(wl, q, k, theta, seg=None):
    # the rotation does not depend on the tile shape (bf16 attention needs
    # head_dim 128; the rotation also runs at 64)
    seg = seg or mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, 64, 64)
    qd, kd = dev(q), dev(k)
    mis.mis_apply_rope(seg, qd, kd, theta)
    torch.cuda.synchronize()
    return host(qd), host(kd), seg


def _check(got, ref, bf16):
    g = oracle.as_f64(got)
    if bf16:
        err = np.abs(g - ref) - (2.0 ** -8 * np.abs(ref) + 1e-5)
        assert err.max() <= 0, f"max excess {err.max():.3e}"
    else:
        assert np.abs(g - ref).max() <= TOL_F32


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_rope_small_batches(dtype, d, theta):
    wl = workloads.from_lengths(f"rope-{dtype}-{d}", [37, 0, 130], [[5, 9, 1], [3, 70], [12] * 6],
                                hq=8, hkv=2, d=d, dtype=dtype, seed=11)
    say(f"[rope] {wl.name} theta={theta} T={wl.total_tokens}")
    q, k, _ = workloads.qkv(wl)
    gq, gk, _ = _gpu_rope(wl, q, k, theta)
    pos = segments_oracle(wl)["pos_id"]
    _check(gq, oracle.rope(q, pos, theta), dtype == "bf16")
    _check(gk, oracle.rope(k, pos, theta), dtype == "bf16")


def test_rope_single_token_request():
    wl = workloads.from_lengths("rope-one", [1], [[]], hq=4, hkv=4, d=128, seed=2)
    q, k, _ = workloads.qkv(wl)
    gq, gk, _ = _gpu_rope(wl, q, k, 1e4)
    assert np.array_equal(gq, q) and np.array_equal(gk, k)  # position 0: identity, bit for bit


def test_rope_single_request_workload_full():
    wl = workloads.config(2)
    say(f"[rope] {wl.name} T={wl.total_tokens}")
    q, k, _ = workloads.qkv(wl)
    gq, gk, _ = _gpu_rope(wl, q, k, 1e6)
    pos = segments_oracle(wl)["pos_id"]
    _check(gq, oracle.rope(q, pos, 1e6), True)
    _check(gk, oracle.rope(k, pos, 1e6), True)


def test_rope_long_prefix_workload_sampled_tokens():
    wl = workloads.config(5)
    say(f"[rope] {wl.name} T={wl.total_tokens}")
    q, k, _ = workloads.qkv(wl)
    gq, gk, _ = _gpu_rope(wl, q, k, 1e6)
    pos = segments_oracle(wl)["pos_id"]
    rng = np.random.default_rng(5)
    rows = np.unique(np.concatenate([rng.integers(0, wl.total_tokens, 1500),
                                     wl.cu_seqlens[1:] - 1, wl.cu_seqlens[:-1] + wl.prefix_lens - 1]))
    _check(gq[rows], oracle.rope(q[rows], pos[rows], 1e6), True)
    _check(gk[rows], oracle.rope(k[rows], pos[rows], 1e6), True)


@pytest.mark.parametrize("dtype,d,tol", [("bf16", 128, TOL_BF16_ATTN), ("f32", 64, TOL_F32)])
def test_mis_with_rope_equals_single_item_scoring(dtype, d, tol):
    wl = workloads.from_lengths(f"rope-sis-{dtype}", [70, 5], [[4, 1, 33, 8], [2, 17]], hq=8, hkv=4, d=d,
                                dtype=dtype, seed=21)
    say(f"[rope+attention] {wl.name}")
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    qd, kd = dev(q), dev(k)
    mis.mis_apply_rope(seg, qd, kd, 1e4)
    o = host(mis.mis_attention_prefill(seg, qd, kd, dev(v), o=nan_like(qd)))
    torch.cuda.synchronize()
    sis = oracle.sis_rope_attention(q, k, v, wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, 1e4)
    assert np.abs(oracle.as_f64(o) - sis).max() <= tol
