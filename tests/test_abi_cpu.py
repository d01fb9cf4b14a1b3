"""C-ABI checks that need no GPU: symbols, size queries, host-side validation.

Every malformed input below is rejected by the host checks before the
library touches the HIP runtime, so nothing here reaches a device.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import item_scoring_attention_amd as mis
from item_scoring_attention_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mis.h")


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(mis_\w+)\s*\(", text, flags=re.M)))


def test_library_loads_and_exports_every_declared_symbol():
    lib = mis.load()
    declared = _declared_functions()
    assert set(declared) >= {"mis_build_segments", "mis_attention_prefill", "mis_score_labels"}
    for name in declared:
        assert hasattr(lib, name), name
        assert name in _lib.SIGNATURES, name
    assert mis.version().startswith("mis-gfx950")


def test_struct_layout_matches_header():
    # 9 int32 fields (padded to 8-byte alignment) then 10 pointers
    assert mis.MisSegments.cu_seqlens.offset == 40
    assert ctypes.sizeof(mis.MisSegments) == 40 + 10 * 8


def _i32(a):
    a = np.ascontiguousarray(np.asarray(a, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def _seg_bytes(cu, n, bm=64, bn=64):
    lib = mis.load()
    a, p = _i32(cu)
    out = ctypes.c_size_t(0)
    rc = lib.mis_segments_bytes(len(a) - 1, p, n, bm, bn, ctypes.byref(out))
    return rc, out.value


def test_segments_bytes_grows_with_size_and_rejects_bad_input():
    rc, small = _seg_bytes([0, 100], 4)
    assert rc == 0 and small > 0
    rc, big = _seg_bytes([0, 100, 5000], 80)
    assert rc == 0 and big > small
    assert _seg_bytes([0, 100], 4, bm=48, bn=24)[0] == mis.MIS_ERR_UNSUPPORTED
    assert _seg_bytes([0, 100], 4, bm=512)[0] == mis.MIS_ERR_UNSUPPORTED
    assert _seg_bytes([1, 100], 4)[0] == mis.MIS_ERR_SEGMENTS
    assert _seg_bytes([0, 100, 100], 4)[0] == mis.MIS_ERR_SEGMENTS
    assert _seg_bytes([0, 100], -1)[0] == mis.MIS_ERR_ARG


def _build(cu, pl, ci, st, bm=64, bn=64, dev=0x1000, dev_bytes=1 << 30):
    """Call mis_build_segments on the host; ``dev`` is never dereferenced for bad metadata."""
    lib = mis.load()
    a, pa = _i32(cu)
    b, pb = _i32(pl)
    c, pc = _i32(ci)
    d, pd = _i32(st)
    out = mis.MisSegments()
    rc = lib.mis_build_segments(len(a) - 1, pa, pb, pc, pd if d.size else None, bm, bn,
                                ctypes.c_void_p(dev), dev_bytes, ctypes.byref(out), None)
    return rc, mis.last_error()


@pytest.mark.parametrize(
    "cu,pl,ci,st,code",
    [
        ([0, 20, 10], [4, 2], [0, 1, 2], [4, 2], mis.MIS_ERR_SEGMENTS),  # cu_seqlens decreasing
        ([0, 20], [4], [0, 2], [5, 10], mis.MIS_ERR_SEGMENTS),  # first item != prefix length
        ([0, 20], [4], [0, 2], [4, 25], mis.MIS_ERR_SEGMENTS),  # item beyond the request
        ([0, 20], [4], [0, 3], [4, 10, 10], mis.MIS_ERR_SEGMENTS),  # empty item
        ([0, 20], [4], [0, 3], [4, 12, 8], mis.MIS_ERR_SEGMENTS),  # out of order
        ([0, 20], [21], [0, 0], [], mis.MIS_ERR_SEGMENTS),  # prefix longer than request
        ([0, 20], [-1], [0, 1], [0], mis.MIS_ERR_SEGMENTS),  # negative prefix
        ([0, 20], [10], [0, 0], [], mis.MIS_ERR_SEGMENTS),  # no items but prefix != length
        ([0, 20], [4], [1, 2], [4], mis.MIS_ERR_SEGMENTS),  # cu_items[0] != 0
        ([0, 20, 30], [4, 3], [0, 2, 1], [4, 9], mis.MIS_ERR_SEGMENTS),  # cu_items decreasing
    ],
)
def test_build_rejects_malformed_metadata(cu, pl, ci, st, code):
    rc, msg = _build(cu, pl, ci, st)
    assert rc == code and msg


def test_build_rejects_null_and_small_buffers():
    rc, _ = _build([0, 20], [4], [0, 2], [4, 10], dev=0)
    assert rc == mis.MIS_ERR_ARG
    rc, msg = _build([0, 20], [4], [0, 2], [4, 10], dev_bytes=16)
    assert rc == mis.MIS_ERR_WORKSPACE and "required" in msg
    rc, _ = _build([0, 20], [4], [0, 2], [4, 10], bm=40)
    assert rc == mis.MIS_ERR_UNSUPPORTED


def test_tile_shape_query():
    assert mis.mis_attention_tile_shape(mis.MIS_BF16, 32, 8, 128) == (64, 64)
    assert mis.mis_attention_tile_shape(mis.MIS_F32, 4, 4, 64) == (64, 64)
    with pytest.raises(ValueError):
        mis.mis_attention_tile_shape(mis.MIS_BF16, 6, 4, 128)
    with pytest.raises(RuntimeError):
        mis.mis_attention_tile_shape(mis.MIS_BF16, 8, 8, 96)
    with pytest.raises(RuntimeError):
        mis.mis_attention_tile_shape(mis.MIS_BF16, 8, 8, 64)


def _fake_seg(n_items=4, tokens=100, bm=64, bn=64):
    s = mis.MisSegments()
    s.num_requests, s.total_tokens, s.total_items = 1, tokens, n_items
    s.block_m, s.block_n, s.num_tiles, s.num_work = bm, bn, 4, 2
    s.work = s.tile_class = s.item_id = s.readout_pos = 0x1000
    return s


def test_attention_argument_errors():
    lib = mis.load()
    s = _fake_seg()
    p = ctypes.c_void_p(0x1000)
    call = lambda seg, q, dt, hq, hkv, d, sc=0.0: lib.mis_attention_prefill(
        seg, q, p, p, p, dt, hq, hkv, d, sc, None)
    assert call(None, p, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), None, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 3, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 4, 80) == mis.MIS_ERR_UNSUPPORTED
    assert call(ctypes.byref(s), p, 7, 8, 4, 128) == mis.MIS_ERR_UNSUPPORTED
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 4, 128, float("nan")) == mis.MIS_ERR_ARG
    s2 = _fake_seg(bm=32)
    assert call(ctypes.byref(s2), p, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_UNSUPPORTED
    # bf16 kernels address a request with 32-bit byte offsets: (T_r + 64) x hq x D x 2 < 4 GiB
    s3 = _fake_seg()
    s3.max_seqlen = 262080  # + 64 = 2^18 rows of 64 heads x 128 dims x 2 bytes = 4 GiB
    assert call(ctypes.byref(s3), p, mis.MIS_BF16, 64, 8, 128) == mis.MIS_ERR_UNSUPPORTED
    assert "4 GiB" in mis.last_error()
    # the item-rows-only entry point runs the same host checks
    call = lambda seg, q, dt, hq, hkv, d, sc=0.0: lib.mis_attention_append(seg, q, p, p, p, dt, hq, hkv, d, sc, None)
    assert call(None, p, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 3, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s2), p, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_UNSUPPORTED
    assert call(ctypes.byref(s3), p, mis.MIS_BF16, 64, 8, 128) == mis.MIS_ERR_UNSUPPORTED


def test_score_argument_errors():
    lib = mis.load()
    s = _fake_seg()
    p = ctypes.c_void_p(0x1000)
    need = mis.mis_score_workspace_bytes(4, 1000, 2, 256, mis.MIS_BF16)
    assert need > 0

    def call(labels, K, ws_bytes=need, H=256, V=1000, dt=mis.MIS_BF16):
        a, pa = _i32(labels)
        return lib.mis_score_labels(ctypes.byref(s), p, H, p, V, dt, pa if a.size else None, K, 0,
                                    p, p, ws_bytes, None)

    assert call([3, 7], 0) == mis.MIS_ERR_LABEL
    assert call([3, 7], 300) == mis.MIS_ERR_LABEL
    assert call([3, 1000], 2) == mis.MIS_ERR_LABEL
    assert call([-1, 5], 2) == mis.MIS_ERR_LABEL
    assert call([3, 7], 2, ws_bytes=need - 1) == mis.MIS_ERR_WORKSPACE
    assert call([3, 7], 2, H=100) == mis.MIS_ERR_UNSUPPORTED
    assert call([3, 7], 2, H=(1 << 22) + 32) == mis.MIS_ERR_UNSUPPORTED  # beyond 32-bit row offsets
    assert call([], 2) == mis.MIS_ERR_ARG
    assert lib.mis_score_labels(None, p, 256, p, 1000, mis.MIS_BF16, None, 2, 0, p, p, need,
                                None) == mis.MIS_ERR_ARG


def test_errors_raise_python_exceptions():
    with pytest.raises(ValueError):
        mis.mis_segments_bytes([0, 10, 5], 0, 64, 64)
    with pytest.raises(RuntimeError):
        mis.mis_segments_bytes([0, 10], 0, 64, 60)
    with pytest.raises(ValueError):
        mis.mis_score_workspace_bytes(4, 1000, 0, 64, mis.MIS_F32)


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="checks the no-device path; a device is visible")
def test_valid_call_without_a_device_reports_hip_error():
    rc, msg = _build([0, 20], [4], [0, 2], [4, 10])
    assert rc == mis.MIS_ERR_HIP and msg


def test_rope_argument_errors():
    # every call below fails its host checks before anything is enqueued (the
    # fake descriptor has no position ids), so no kernel ever sees its pointers
    lib = mis.load()
    s = _fake_seg()
    p = ctypes.c_void_p(0x1000)
    call = lambda seg, q, dt, hq, hkv, d, theta=1e4: lib.mis_apply_rope(seg, q, p, dt, hq, hkv, d, theta, None)
    assert call(None, p, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_ARG
    assert lib.mis_apply_rope(ctypes.byref(s), p, None, mis.MIS_BF16, 8, 4, 128, 1e4, None) == mis.MIS_ERR_ARG
    assert "k must be" in mis.last_error()
    # q may be NULL (K rotated alone): the checks then stop at the missing position ids
    assert call(ctypes.byref(s), None, mis.MIS_BF16, 8, 4, 128) == mis.MIS_ERR_ARG
    assert "not a built segment" in mis.last_error()
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 3, 128) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 4, 80) == mis.MIS_ERR_UNSUPPORTED
    assert call(ctypes.byref(s), p, 7, 8, 4, 128) == mis.MIS_ERR_UNSUPPORTED
    for theta in (0.0, -5.0, float("nan"), float("inf")):
        assert call(ctypes.byref(s), p, mis.MIS_BF16, 8, 4, 128, theta) == mis.MIS_ERR_ARG
    assert call(ctypes.byref(s), p, mis.MIS_F32, 8, 4, 64) == mis.MIS_ERR_ARG  # no position ids
    assert "not a built segment" in mis.last_error()


def test_rope_table_and_fused_attention_argument_errors():
    lib = mis.load()
    out = ctypes.c_size_t(0)
    assert lib.mis_rope_table_bytes(100, 128, ctypes.byref(out)) == mis.MIS_OK and out.value == 100 * 128 * 4
    assert lib.mis_rope_table_bytes(7, 64, ctypes.byref(out)) == mis.MIS_OK and out.value == 7 * 64 * 4
    assert lib.mis_rope_table_bytes(0, 128, ctypes.byref(out)) == mis.MIS_ERR_ARG
    assert lib.mis_rope_table_bytes(10, 96, ctypes.byref(out)) == mis.MIS_ERR_UNSUPPORTED
    assert lib.mis_rope_table_bytes(10, 128, None) == mis.MIS_ERR_ARG
    assert mis.mis_rope_table_bytes(33, 128) == 33 * 128 * 4
    p = ctypes.c_void_p(0x1000)
    # rejected before anything is enqueued
    assert lib.mis_rope_table(10, 128, 1e4, None, 5120, None) == mis.MIS_ERR_ARG
    assert lib.mis_rope_table(10, 128, 1e4, p, 5119, None) == mis.MIS_ERR_ARG
    for theta in (0.0, -1.0, float("nan"), float("inf")):
        assert lib.mis_rope_table(10, 128, theta, p, 5120, None) == mis.MIS_ERR_ARG
    s = _fake_seg()
    s.max_seqlen = 100
    for fn in (lib.mis_attention_prefill_rope, lib.mis_attention_append_rope):
        call = lambda dt, table, npos, d=128, seg=s: fn(ctypes.byref(seg), p, p, p, p, dt, 8, 4, d, 0.0, table,
                                                        npos, None)
        assert call(mis.MIS_BF16, None, 100) == mis.MIS_ERR_ARG
        assert "rope_table" in mis.last_error()
        assert call(mis.MIS_BF16, p, 99) == mis.MIS_ERR_ARG
        assert "short" in mis.last_error()
        bm, bn = mis.mis_attention_tile_shape(mis.MIS_F32, 8, 4, 64)
        s32 = _fake_seg(bm=bm, bn=bn)
        s32.max_seqlen = 100
        assert call(mis.MIS_F32, p, 100, d=64, seg=s32) == mis.MIS_ERR_UNSUPPORTED
        assert "bf16 only" in mis.last_error()


def test_score_at_argument_errors():
    # positions and labels are checked on the host before anything is enqueued
    lib = mis.load()
    p = ctypes.c_void_p(0x1000)
    lab = np.asarray([3, 7], dtype=np.int32)
    def call(pos, nrows, ntok=100, labels=lab, k=2, ws_bytes=1 << 30, dt=mis.MIS_BF16, h=256):
        pos = np.asarray(pos, dtype=np.int32)
        labels = np.asarray(labels, dtype=np.int32)
        return lib.mis_score_labels_at(pos.ctypes.data if pos.size else None, nrows, ntok, p, h, p, 1000, dt,
                                       labels.ctypes.data, k, 0, p, p, ws_bytes, None)
    assert call([5, 100], 2) == mis.MIS_ERR_ARG and "outside" in mis.last_error()
    assert call([-1], 1) == mis.MIS_ERR_ARG
    assert call([5], 1, labels=[3, 1000]) == mis.MIS_ERR_LABEL
    assert call([5], 1, k=0) == mis.MIS_ERR_LABEL
    assert call([5], 1, ws_bytes=16) == mis.MIS_ERR_WORKSPACE
    assert call([5], 1, h=100) == mis.MIS_ERR_UNSUPPORTED
    assert call([5], -1) == mis.MIS_ERR_ARG
    assert call([], 0) == mis.MIS_OK  # nothing to score: validated, nothing enqueued


def test_kernel_choice_names_and_rejects_unknown():
    mis.set_kernel_choice()
    with pytest.raises(ValueError, match="unknown attention kernel choice"):
        mis.set_kernel_choice(attention="fastest")
    for bad in ("wide7", "persist2", "persist6", "persist8", "narrow2"):
        with pytest.raises(ValueError, match="unknown scoring kernel choice"):
            mis.set_kernel_choice(score=bad)
    bf16 = mis.MIS_BF16
    try:
        # scoring: the shapes of the five workloads, then forced variants
        assert mis.score_kernel_name(64, 1024, bf16) == "score_lds_kernel<2, 3>"
        assert mis.score_kernel_name(300, 4096, bf16) == "score_persist_kernel<5, 3>"
        assert mis.score_kernel_name(1024, 8192, bf16) == "score_persist_kernel<4, 3>"
        assert mis.score_kernel_name(6400, 1024, bf16) == "score_persist_kernel<5, 3>"
        assert mis.score_kernel_name(80, 64, bf16) == "score_wide_kernel<3, 3>"  # H < 128
        assert mis.score_kernel_name(4, 256, mis.MIS_F32) == "score_f32_kernel"
        assert mis.score_kernel_name(200, 96, bf16) == "score_bf16_kernel<4>"
        mis.set_kernel_choice(score="persist")
        assert mis.score_kernel_name(64, 1024, bf16) == "score_persist_kernel<3, 3>"  # 96 slots, the fewest
        assert mis.score_kernel_name(128, 1024, bf16) == "score_persist_kernel<4, 3>"  # no padding
        assert mis.score_kernel_name(300, 4096, bf16) == "score_persist_kernel<5, 3>"
        mis.set_kernel_choice(score="persist5")
        assert mis.score_kernel_name(1024, 8192, bf16) == "score_persist_kernel<5, 3>"
        mis.set_kernel_choice(score="persist3")
        assert mis.score_kernel_name(64, 1024, bf16) == "score_persist_kernel<3, 3>"
        assert mis.score_kernel_name(80, 64, bf16) == "score_wide_kernel<3, 3>"  # H < 128: wide tiles
        mis.set_kernel_choice(score="wide4")
        assert mis.score_kernel_name(64, 1024, bf16) == "score_wide_kernel<4, 3>"
        mis.set_kernel_choice(score="narrow")
        assert mis.score_kernel_name(1024, 8192, bf16) == "score_lds_kernel<4, 2>"
        assert mis.score_kernel_name(200, 96, bf16) == "score_bf16_kernel<4>"  # H % 64 != 0

        # attention: picked from the segment counts (no device memory is read)
        seg = mis.Segments(mis.MisSegments(num_requests=4, total_tokens=115712, block_m=64, block_n=64,
                                           num_work=1808, num_visits=1808 * 259), None)
        mis.set_kernel_choice()
        assert mis.attention_kernel_name(seg, bf16, 64, 8, 128) == "attn_pipe_kernel<4, 1>"
        assert mis.attention_kernel_name(seg, bf16, 16, 8, 128) == "attn_pipe_kernel<2, 1>"
        assert mis.attention_kernel_name(seg, bf16, 12, 4, 128) == "attn_dma_kernel<2, 1>"
        assert mis.attention_kernel_name(seg, mis.MIS_F32, 4, 4, 64) == "attn_f32_kernel"
        short = mis.Segments(mis.MisSegments(num_requests=1, total_tokens=4160, block_m=64, block_n=64,
                                             num_work=65, num_visits=65 * 20), None)
        assert mis.attention_kernel_name(short, bf16, 64, 8, 128) == "attn_pipe_kernel<2, 2>"
        # groups of 2: 64 rows per wave from 20 visits per query tile on
        assert mis.attention_kernel_name(short, bf16, 16, 8, 128) == "attn_pipe_kernel<2, 1>"
        few = mis.Segments(mis.MisSegments(num_requests=1, total_tokens=4160, block_m=64, block_n=64,
                                           num_work=65, num_visits=65 * 20 - 1), None)
        assert mis.attention_kernel_name(few, bf16, 16, 8, 128) == "attn_pipe_kernel<2, 2>"
        mis.set_kernel_choice(attention="pipe")
        assert mis.attention_kernel_name(short, bf16, 16, 8, 128) == "attn_pipe_kernel<2, 1>"
        assert mis.attention_kernel_name(short, bf16, 12, 4, 128) == "attn_dma_kernel<2, 1>"
        mis.set_kernel_choice(attention="pipe2")
        assert mis.attention_kernel_name(short, bf16, 64, 8, 128) == "attn_pipe_kernel<2, 1>"
        mis.set_kernel_choice(attention="classic")
        assert mis.attention_kernel_name(short, bf16, 64, 8, 128) == "attn_dma_kernel<2, 2>"
        with pytest.raises(ValueError):
            mis.attention_kernel_name(short, bf16, 64, 8, 64)  # bf16 is built for head_dim 128
    finally:
        mis.set_kernel_choice()


def test_noalloc_scoring_rejects_bad_arguments_on_the_host():
    lib = mis.load()
    seg = mis.MisSegments(num_requests=1, total_tokens=10, total_items=2000, block_m=64, block_n=64,
                          readout_pos=0x1000)
    lab, lp = _i32([1, 2])
    # partials of 2000 items at a 151936-token vocabulary exceed the 16 MiB scratch
    rc = lib.mis_score_labels_noalloc(ctypes.byref(seg), ctypes.c_void_p(0x1000), 64, ctypes.c_void_p(0x1000),
                                      151936, mis.MIS_BF16, lp, 2, 0, ctypes.c_void_p(0x1000), None)
    assert rc == mis.MIS_ERR_WORKSPACE and "scratch" in mis.last_error()
    rc = lib.mis_score_labels_noalloc(ctypes.byref(seg), ctypes.c_void_p(0x1000), 64, ctypes.c_void_p(0x1000),
                                      1000, mis.MIS_BF16, _i32([1000])[1], 1, 0, ctypes.c_void_p(0x1000), None)
    assert rc == mis.MIS_ERR_LABEL
    rc = lib.mis_score_labels_noalloc(ctypes.byref(seg), ctypes.c_void_p(0x1000), 64, ctypes.c_void_p(0x1000),
                                      1000, mis.MIS_BF16, lp, 2, 0, None, None)
    assert rc == mis.MIS_ERR_ARG
