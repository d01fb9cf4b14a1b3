"""Build ``libmis.so`` (the C-ABI library) for gfx950 with hipcc, in-tree.

Usage: ``python -m item_scoring_attention_amd.build`` (or ``build()``). Every
call recompiles all sources; objects go to ``_build/`` next to this file and
the shared libraries to the package directory: ``libmis.so`` (the C ABI) and
``libmis_probe.so`` (the MFMA-rate probe the benchmark prices against; not
part of the ABI).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libmis.so")
PROBE_LIB = os.path.join(PKG, "libmis_probe.so")
ARCH = "gfx950"

SOURCES = ["abi.cpp", "segments.hip", "rope.hip", "attn_f32.hip", "attn_bf16.hip", "attn_bf16_pipe.hip",
           "score.hip"]
PROBE_SOURCES = ["probe.hip"]

# Per-source extra flags. The attention kernels keep their MFMA accumulators
# in VGPRs: with the default heuristic the allocator parks them in AGPRs and
# copies them back on every key tile.
EXTRA_FLAGS = {"attn_bf16.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}

# -packed-fp32-ops keeps hipcc from forming packed fp32 VALU instructions.
# The host pass warns that it does not know the feature; that is harmless.
FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    f"-I{INCLUDE}",
    f"-I{CSRC}",
]


def _hipcc() -> str:
    exe = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(exe):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return exe


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [_hipcc(), *FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    msgs = "\n".join(
        ln for ln in (res.stdout + res.stderr).splitlines()
        if "packed-fp32-ops" not in ln
    )
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{msgs}")
    if msgs.strip() and verbose:
        print(msgs, flush=True)
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [_hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stdout}{res.stderr}")
    # A kernel template whose host-side instantiation fails leaves its launch
    # stub undefined without a compile error; refuse such a library.
    nm = shutil.which("nm")
    if nm:
        und = subprocess.run([nm, "-u", tmp], capture_output=True, text=True).stdout
        bad = [ln.split()[-1] for ln in und.splitlines() if "__device_stub__" in ln]
        if bad:
            raise RuntimeError(f"undefined kernel launch stubs in {tmp}: {bad}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    """Compile every source for gfx950 and link ``libmis.so`` and
    ``libmis_probe.so``; return the path of ``libmis.so``."""
    t0 = time.time()
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + PROBE_SOURCES
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 1)) as ex:
        objs = dict(zip(srcs, ex.map(lambda s: _compile(s, verbose), srcs)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in PROBE_SOURCES], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB} in {time.time() - t0:.1f}s", flush=True)
    return LIB


if __name__ == "__main__":
    build(verbose="-q" not in sys.argv)
