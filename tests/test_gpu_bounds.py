"""Rows past a request's end are never read by the bf16 attention kernels.

Each staged K/V tile is loaded through a buffer descriptor whose range ends
at the request's last key; a lane whose row lies past that end must read
nothing. The inputs here sit in allocations with 64 extra rows of bf16 NaN
after the last token, and the kernels get views of the first T rows, so any
read past the end puts a NaN into the output (a zero probability times a NaN
value is NaN). Every access stays inside the allocation. The last request's
length is 1 or 9 modulo 64, so its last key tile is mostly past the end.
"""
import numpy as np
import pytest
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads
from gpu_common import TOL_BF16_ATTN, build, dev, host, nan_like, say, segments_oracle

pytestmark = pytest.mark.gpu

PAD = 64


@pytest.fixture(autouse=True, params=["auto", "pipe", "pipe2", "pipe32", "classic"])
def attention_kernel(request):
    """Each bf16 attention kernel, forced, and the one chosen by shape."""
    mis.set_kernel_choice(attention=request.param)
    yield request.param
    mis.set_kernel_choice()


def _nan_padded(x: np.ndarray) -> torch.Tensor:
    buf = np.full((x.shape[0] + PAD,) + x.shape[1:], workloads.NAN_BF16, dtype=np.uint16)
    buf[: x.shape[0]] = x
    return dev(buf)


@pytest.mark.parametrize("prefix,items,hq,hkv", [
    ([60], [[20, 40, 9]], 8, 4),                    # T = 129 = 2 * 64 + 1, group of 2
    ([130, 60], [[9, 33, 1], [20, 40, 9]], 16, 4),  # last request 129 tokens, group of 4
    ([300, 101], [[12] * 5, [30, 6]], 8, 2),        # last request 137 = 2 * 64 + 9, group of 4
    ([2000], [[37] * 5], 8, 4),                     # T = 2185 = 34 * 64 + 9, long visit lists
])
def test_rows_past_the_end_are_not_read(prefix, items, hq, hkv):
    wl = workloads.from_lengths("past-end", prefix, items, hq=hq, hkv=hkv, d=128, seed=sum(prefix))
    T = wl.total_tokens
    say(f"[bounds] T={T} (T mod 64 = {T % 64}) hq={hq} hkv={hkv}")
    q, k, v = workloads.qkv(wl)
    qf, kf, vf = _nan_padded(q), _nan_padded(k), _nan_padded(v)
    qd, kd, vd = qf[:T], kf[:T], vf[:T]
    assert qd.is_contiguous() and qd.data_ptr() == qf.data_ptr()
    seg = build(wl)
    o = nan_like(qd)
    mis.mis_attention_prefill(seg, qd, kd, vd, o=o)
    torch.cuda.synchronize()
    got = oracle.as_f64(host(o))
    assert np.isfinite(got).all()
    ref = oracle.attention(q, k, v, wl.cu_seqlens, segments_oracle(wl)["item_id"])
    e = float(np.abs(got - ref).max())
    say(f"  max abs err {e:.3e}")
    assert e <= TOL_BF16_ATTN
    # the padding itself is untouched
    assert torch.isnan(kf[T:].float()).all() and torch.isnan(vf[T:].float()).all()
