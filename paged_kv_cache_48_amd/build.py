"""Build libpaged_attn.so in-tree with hipcc for gfx950.

Usage: ``python -m paged_kv_cache_48_amd.build`` (or ``build()`` from Python).
Objects go to ``_build/`` at the repository root; the library is written next
to this file so the Python binding finds it.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
LIB_PATH = os.path.join(HERE, "libpaged_attn.so")
SOURCES = ["api.hip", "cache_ops.hip", "decode.hip", "prefill.hip", "mixed.hip"]
# per-source extra flags: the attention kernels keep their MFMA results in
# VGPRs (the softmax reads the scores and rescales the accumulators on the
# VALU, which would otherwise copy them out of the accumulation registers on
# every tile)
EXTRA = {src: ["-mllvm", "-amdgpu-mfma-vgpr-form"] for src in ("decode.hip", "prefill.hip", "mixed.hip")}

# -packed-fp32-ops: keep the compiler from emitting packed fp32 VALU ops.
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc() -> str:
    env = os.environ.get("HIPCC")
    if env:
        return env
    for cand in ("/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (set HIPCC)")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the packed-fp32 feature; that is expected
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile every HIP source for gfx950 and link libpaged_attn.so.  Always rebuilds."""
    cc = hipcc()
    objdir = os.path.join(ROOT, "_build")
    os.makedirs(objdir, exist_ok=True)
    objs = []
    cmds = []
    for src in SOURCES:
        obj = os.path.join(objdir, src.replace(".hip", ".o"))
        objs.append(obj)
        cmds.append([cc, *FLAGS, *EXTRA.get(src, []), "-c", os.path.join(HERE, "csrc", src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        list(ex.map(lambda c: _run(c, verbose), cmds))
    tmp = LIB_PATH + ".tmp"
    _run([cc, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
