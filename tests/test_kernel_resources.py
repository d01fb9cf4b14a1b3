"""Register and LDS budgets of the gfx950 kernels, from the compiler's own
kernel metadata for this repository's sources (device assembly, no GPU).

The occupancy each kernel is designed for rests on these numbers: the
32-row attention loop and the plain attention loop need at most 256
registers (VGPRs + AGPRs) for two waves per SIMD, their 2-head workgroups at
most 80 KB of LDS for two workgroups per CU, and no kernel may spill. A
compiler or generator change that breaks one of them would only show up as
a slowdown on the GPU, so it is checked here.
"""
import os
import subprocess
import tempfile

import pytest
import yaml

from item_scoring_attention_amd import build as B


def _kernels(src: str) -> dict:
    try:
        hipcc = B._hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        flags = [f for f in B.FLAGS if f != "-fPIC"]
        cmd = [hipcc, *flags, *B.EXTRA_FLAGS.get(src, []), "-x", "hip", "--offload-device-only", "-S",
               os.path.join(B.CSRC, src), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert res.returncode == 0, res.stderr[-2000:]
        text = open(out).read()
    meta = text[text.index("amdhsa.kernels:"):]
    meta = meta[:meta.index("\n...")]
    return {k[".name"]: k for k in yaml.safe_load(meta)["amdhsa.kernels"]}


@pytest.fixture(scope="module")
def kernels():
    ks = {}
    for src in ("attn_bf16.hip", "attn_bf16_pipe.hip", "score.hip"):
        ks.update(_kernels(src))
    return ks


def _find(kernels, fragment):
    hits = [k for name, k in kernels.items() if fragment in name]
    assert hits, f"no kernel matching {fragment}"
    return hits


def test_no_kernel_spills(kernels):
    # No register goes to memory. A few scalar registers parked in vector
    # register lanes (v_writelane / v_readlane, no scratch) are allowed.
    for name, k in kernels.items():
        assert k[".vgpr_spill_count"] == 0, name
        assert k[".private_segment_fixed_size"] == 0, name
        assert k[".sgpr_spill_count"] <= 8, name


def test_two_waves_per_simd_kernels_fit_256_registers(kernels):
    # attn_pipe_kernel<2, 2> (32 rows per wave) and attn_dma_kernel<2, 2>
    for frag in ("attn_pipe_kernelILi2ELi2E", "attn_dma_kernelILi2ELi2E"):
        for k in _find(kernels, frag):
            assert k[".vgpr_count"] <= 256, (frag, k[".vgpr_count"])


def test_two_workgroups_per_cu_fit_the_lds(kernels):
    for frag in ("attn_pipe_kernelILi2ELi2E", "attn_pipe_kernelILi2ELi1E", "attn_dma_kernelILi2E"):
        for k in _find(kernels, frag):
            assert 2 * k[".group_segment_fixed_size"] <= 160 * 1024, frag


def test_single_workgroup_kernels_fit_the_lds(kernels):
    for frag in ("attn_pipe_kernelILi4ELi1E", "score_wide_kernel", "score_lds_kernel", "score_persist_kernel"):
        for k in _find(kernels, frag):
            assert k[".group_segment_fixed_size"] <= 160 * 1024, frag
