"""mis_build_segments accepts exactly the metadata its header allows.

Random packed batches, each either well formed or broken in one of the ways
the header's rules forbid, go through the C ABI's host checks; the expected
verdict comes from a plain restatement of those rules in Python (cu_seqlens
from 0, every request at least one token; 0 <= Lq <= T per request;
cu_items from 0 and non-decreasing, N = cu_items[B]; a request's first item starts
at Lq, starts strictly increase and stay inside the request; a request with
no items is all prefix). Well-formed metadata passes every check and, with no
device visible, stops at the HIP runtime; broken metadata is refused before
anything else. CPU only: the test is skipped where a device is visible,
since a well-formed call would then launch the builder on a fake buffer.
"""
import ctypes

import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import item_scoring_attention_amd as mis


def _gpu_visible():
    try:
        import torch

        return torch.cuda.is_available()
    except Exception:
        return False


pytestmark = pytest.mark.skipif(_gpu_visible(), reason="needs the no-device path of the host checks")


def _valid(cu, pl, ci, starts) -> bool:
    B = len(cu) - 1
    if B < 1 or len(pl) != B or len(ci) != B + 1 or cu[0] != 0 or ci[0] != 0:
        return False
    if any(cu[r + 1] - cu[r] < 1 for r in range(B)):
        return False
    if any(ci[r + 1] < ci[r] for r in range(B)):
        return False
    # N is cu_items[B] (the C ABI cannot see the array's length)
    starts = list(starts[:ci[B]]) + [0] * max(0, ci[B] - len(starts))
    for r in range(B):
        T = cu[r + 1] - cu[r]
        if not 0 <= pl[r] <= T:
            return False
        s = starts[ci[r]:ci[r + 1]]
        if not s:
            if pl[r] != T:
                return False
            continue
        if s[0] != pl[r] or any(b <= a for a, b in zip(s, s[1:])) or s[-1] >= T:
            return False
    return True


@st.composite
def batches(draw):
    B = draw(st.integers(1, 4))
    cu, pl, ci, starts = [0], [], [0], []
    for _ in range(B):
        n_items = draw(st.integers(0, 6))
        lq = draw(st.integers(0, 40))
        lens = [draw(st.integers(1, 9)) for _ in range(n_items)]
        T = lq + sum(lens) if n_items else max(lq, 1)
        if not n_items:
            lq = T
        pl.append(lq)
        off = lq
        for ln in lens:
            starts.append(off)
            off += ln
        cu.append(cu[-1] + T)
        ci.append(len(starts))
    mutation = draw(st.sampled_from(["none", "none", "cu0", "cu_down", "empty_request", "prefix_long",
                                     "prefix_neg", "first_start", "repeat_start", "start_out", "ci0",
                                     "ci_down", "ci_end", "no_items_prefix"]))
    r = draw(st.integers(0, B - 1))
    if mutation == "cu0":
        cu[0] = 1
    elif mutation == "cu_down" and B > 1:
        cu[r + 1] = cu[r] - 1
    elif mutation == "empty_request":
        delta = cu[r + 1] - cu[r]
        cu = cu[:r + 1] + [c - delta for c in cu[r + 1:]]
    elif mutation == "prefix_long":
        pl[r] = cu[r + 1] - cu[r] + 1
    elif mutation == "prefix_neg":
        pl[r] = -1
    elif mutation == "first_start" and ci[r + 1] > ci[r]:
        starts[ci[r]] += 1
    elif mutation == "repeat_start" and ci[r + 1] - ci[r] >= 2:
        starts[ci[r] + 1] = starts[ci[r]]
    elif mutation == "start_out" and ci[r + 1] > ci[r]:
        starts[ci[r + 1] - 1] = cu[r + 1] - cu[r]
    elif mutation == "ci0":
        ci[0] = 1
    elif mutation == "ci_down" and B > 1 and ci[r + 1] > 0:
        ci[r + 1] = ci[r] - 1 if ci[r] > 0 else ci[r + 1]
    elif mutation == "ci_end" and starts:
        ci[-1] -= 1
    elif mutation == "no_items_prefix" and ci[r + 1] == ci[r] and cu[r + 1] - cu[r] > 1:
        pl[r] -= 1
    return cu, pl, ci, starts


def _i32(x):
    a = np.ascontiguousarray(np.asarray(x, dtype=np.int32))
    return a, a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


@settings(max_examples=400, deadline=None, suppress_health_check=[HealthCheck.too_slow])
@given(batches())
def test_host_checks_accept_exactly_the_header_rules(batch):
    cu, pl, ci, starts = batch
    lib = mis.load()
    a, pa = _i32(cu)
    b, pb = _i32(pl)
    c, pc = _i32(ci)
    n = max(int(ci[-1]), len(starts), 0)
    d, pd = _i32(starts + [0] * (n - len(starts)))  # the library may read cu_items[B] starts
    out = mis.MisSegments()
    rc = lib.mis_build_segments(len(cu) - 1, pa, pb, pc, pd if d.size else None, 64, 64, ctypes.c_void_p(0x1000),
                                1 << 30, ctypes.byref(out), None)
    if _valid(cu, pl, ci, starts):
        assert rc == mis.MIS_ERR_HIP, (rc, mis.last_error(), batch)  # every check passed; no device to run on
    else:
        assert rc in (mis.MIS_ERR_SEGMENTS, mis.MIS_ERR_ARG), (rc, mis.last_error(), batch)
