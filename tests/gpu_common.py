"""Helpers shared by the GPU parity tests: uploads, library calls, row sampling.

Inputs come from ``workloads`` (seeded); expected values come from
``oracle`` only. The library is called through its C ABI binding.
"""
import sys

import numpy as np
import torch

import item_scoring_attention_amd as mis
import oracle
import workloads

# Tolerances: max abs error (fp32 workloads 1e-4; bf16 with fp32 accumulation
# 2e-2 on attention outputs and 1e-2 on label log-probs).
TOL_F32 = 1e-4
TOL_BF16_ATTN = 2e-2
TOL_BF16_SCORE = 1e-2


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def dev(x: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor (uint16 arrays are bf16 bit patterns)."""
    if x.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(x)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    """device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def segments_oracle(wl):
    return oracle.build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts)


def build(wl, dtype=None):
    dt = mis.MIS_BF16 if (dtype or wl.dtype) == "bf16" else mis.MIS_F32
    bm, bn = mis.mis_attention_tile_shape(dt, wl.hq, wl.hkv, wl.d)
    seg = mis.mis_build_segments(wl.cu_seqlens, wl.prefix_lens, wl.cu_items, wl.item_starts, bm, bn)
    return seg


def nan_like(t: torch.Tensor) -> torch.Tensor:
    """A tensor shaped like ``t`` filled with NaN, so an output element that a
    kernel never writes shows up as NaN instead of stale finite memory."""
    return torch.full_like(t, float("nan"))


def attention(wl, seg, q, k, v, scale=0.0):
    qd = dev(q)
    o = nan_like(qd)
    mis.mis_attention_prefill(seg, qd, dev(k), dev(v), o=o, softmax_scale=scale)
    torch.cuda.synchronize()
    return o


_CACHE = {}


def cached(key, fn):
    """Compute ``fn()`` once per test session (oracle results and inputs of the
    large workloads, shared by every kernel a test is parametrised over)."""
    if key not in _CACHE:
        _CACHE[key] = fn()
    return _CACHE[key]


def tile_rows(wl, block_m=64, extra_per_tile=0, seed=0):
    """Packed query rows covering every query tile of every request: the
    tile's first and last row (the last row sees the most keys of the tile)
    plus ``extra_per_tile`` random rows of the tile."""
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(wl.num_requests):
        a, b = int(wl.cu_seqlens[r]), int(wl.cu_seqlens[r + 1])
        for j0 in range(a, b, block_m):
            j1 = min(j0 + block_m, b)
            rows += [j0, j1 - 1]
            if extra_per_tile:
                rows += rng.integers(j0, j1, size=extra_per_tile).tolist()
    return np.unique(np.asarray(rows, dtype=np.int64))


def hidden_with_sentinels(wl, readout_pos):
    """[T, H] hidden states: N(0,1) rows at the readout positions, NaN elsewhere."""
    vals = workloads.readout_values(wl)
    if wl.dtype == "bf16":
        hid = np.full((wl.total_tokens, wl.hidden), workloads.NAN_BF16, dtype=np.uint16)
    else:
        hid = np.full((wl.total_tokens, wl.hidden), np.nan, dtype=np.float32)
    hid[np.asarray(readout_pos)] = vals
    return hid
