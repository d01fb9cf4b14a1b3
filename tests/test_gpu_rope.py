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


# ------------------------------------------------ Q rotated inside attention

KERNELS = ["auto", "pipe", "pipe2", "pipe32", "classic"]


def _fits(choice, wl):
    gsz = wl.hq // wl.hkv
    if choice == "pipe":
        return gsz % 4 == 0
    if choice in ("pipe2", "pipe32"):
        return gsz % 2 == 0
    return True


def test_rope_table_values():
    """cos and sin of p * theta^(-2i/D) for every position and pair: the
    oracle's rotation of the unit vector (1, 0) at position p gives them."""
    for d, theta in ((128, 1e6), (64, 1e4)):
        P = 3000
        t = mis.mis_rope_table(P, d, theta)
        torch.cuda.synchronize()
        got = host(t).astype(np.float64).reshape(P, d // 2, 2)
        unit = np.zeros((P, 1, d), dtype=np.float32)
        unit[:, 0, : d // 2] = 1.0
        rot = oracle.rope(unit, np.arange(P), theta)[:, 0, :]  # (cos, sin) of each pair's angle
        assert np.abs(got[:, :, 0] - rot[:, : d // 2]).max() <= 1e-6
        assert np.abs(got[:, :, 1] - rot[:, d // 2:]).max() <= 1e-6


def _fused_vs_separate(wl, choice, theta=1e6, append=False):
    """Fused: K rotated alone, Q rotated by the attention kernel. Separate:
    both rotated by the rotation pass, then the plain attention call. The
    outputs must agree bit for bit, and the caller's Q stay untouched."""
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    table = mis.mis_rope_table(seg.max_seqlen, wl.d, theta)
    mis.set_kernel_choice(attention=choice)
    try:
        qd, kd, vd = dev(q), dev(k), dev(v)
        mis.mis_apply_rope(seg, None, kd, theta)
        o_f = nan_like(qd)
        if append:
            mis.mis_attention_append_rope(seg, qd, kd, vd, o_f, table)
        else:
            mis.mis_attention_prefill_rope(seg, qd, kd, vd, table, o=o_f)
        q2, k2 = dev(q), dev(k)
        mis.mis_apply_rope(seg, q2, k2, theta)
        o_s = nan_like(qd)
        if append:
            mis.mis_attention_append(seg, q2, k2, vd, o_s)
        else:
            mis.mis_attention_prefill(seg, q2, k2, vd, o=o_s)
        torch.cuda.synchronize()
    finally:
        mis.set_kernel_choice()
    assert np.array_equal(host(qd), q), "q was modified"
    assert np.array_equal(host(kd), host(k2)), "K rotated alone differs from K rotated with Q"
    of, os_ = host(o_f), host(o_s)
    if append:
        items = segments_oracle(wl)["item_id"] >= 0
        of, os_ = of[items], os_[items]
    assert np.array_equal(of, os_), f"{choice}: fused and separate rotation differ"
    assert np.isfinite(oracle.as_f64(of)).all()
    return q, k, v, of


@pytest.mark.parametrize("choice", KERNELS)
def test_fused_rope_small_shapes(choice):
    for wl in (workloads.from_lengths("frope-gqa4", [70, 5, 130], [[4, 1, 33, 8], [2, 17], [20] * 5],
                                      hq=16, hkv=4, d=128, seed=31),
               workloads.from_lengths("frope-gqa2", [200, 0], [[3, 65, 9], [4, 4]], hq=8, hkv=4, d=128, seed=32),
               workloads.from_lengths("frope-mha", [33], [[7, 7, 40]], hq=4, hkv=4, d=128, seed=33)):
        if not _fits(choice, wl):
            continue
        say(f"[fused rope] {wl.name} {choice}")
        q, k, v, o = _fused_vs_separate(wl, choice)
        sis = oracle.sis_rope_attention(q, k, v, wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, 1e6)
        assert np.abs(oracle.as_f64(o) - sis).max() <= TOL_BF16_ATTN


@pytest.mark.parametrize("choice", KERNELS)
def test_fused_rope_single_request_workload(choice):
    wl = workloads.config(2)
    say(f"[fused rope] {wl.name} {choice}")
    _fused_vs_separate(wl, choice)


@pytest.mark.parametrize("choice", ["auto", "pipe32"])
def test_fused_rope_append(choice):
    wl = workloads.config(2)
    say(f"[fused rope append] {wl.name} {choice}")
    _fused_vs_separate(wl, choice, append=True)


def test_fused_rope_long_prefix_workload():
    wl = workloads.config(5)
    say(f"[fused rope] {wl.name}")
    _fused_vs_separate(wl, "auto")


def test_fused_rope_rejects_short_table_and_f32():
    wl = workloads.from_lengths("frope-err", [40], [[5, 6]], hq=8, hkv=4, d=128, seed=34)
    q, k, v = workloads.qkv(wl)
    seg = build(wl)
    qd, kd, vd = dev(q), dev(k), dev(v)
    short = mis.mis_rope_table(seg.max_seqlen - 1, 128, 1e4)
    with pytest.raises(ValueError, match="short"):
        mis.mis_attention_prefill_rope(seg, qd, kd, vd, short)
    wl32 = workloads.from_lengths("frope-f32", [40], [[5, 6]], hq=8, hkv=4, d=64, dtype="f32", seed=35)
    q32, k32, v32 = workloads.qkv(wl32)
    seg32 = build(wl32)
    with pytest.raises(mis.MisError):
        mis.mis_attention_prefill_rope(seg32, dev(q32), dev(k32), dev(v32), mis.mis_rope_table(100, 64, 1e4))
