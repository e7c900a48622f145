"""Build libqift.so (the HIP kernels and the C ABI) in-tree for gfx950.

    python -m bit_quantized_fwht_amd.build        # or build() from Python

hipcc cross-compiles without a GPU. The library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libqift.so")

SOURCES = ["rotate_quant.hip", "kv4.hip", "kv4_attention.hip", "gptq.hip", "linear_decode.hip",
           "linear_prefill.hip", "measure.hip", "api.cpp"]

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # no silent a*b+c fusion: the parity contract fixes the float32 steps
    "-ffp-contract=off",
    # packed fp32 instructions stay off (compiler-generated v_pk_* forms
    # are avoided in all HIP code of this library)
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libqift.so)")


# per-source flags: the KV4 kernels keep their matrix-core results in
# ordinary vector registers (the accumulation registers would need one extra
# move per value, about a tenth of that kernel's vector instructions)
SOURCE_FLAGS = {"kv4.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}

BUILD_DIR = os.path.join(ROOT, "_build")


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose: bool = False, extra_flags=None, jobs: int = 8) -> str:
    """Compile every source to an object (in parallel), then link libqift.so."""
    from concurrent.futures import ThreadPoolExecutor

    os.makedirs(BUILD_DIR, exist_ok=True)
    objs, cmds = [], []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        flags = [f for f in HIPCC_FLAGS if f != "-shared"]
        cmds.append([hipcc(), *flags, *SOURCE_FLAGS.get(src, []), *(extra_flags or []), "-I", INCLUDE,
                     "-I", CSRC, "-c", "-o", obj, os.path.join(CSRC, src)])
        objs.append(obj)
    with ThreadPoolExecutor(max_workers=max(1, min(jobs, len(cmds)))) as ex:
        results = list(ex.map(lambda c: _run(c, verbose), cmds))
    for cmd, res in zip(cmds, results):
        if res.returncode != 0:
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc failed on {cmd[-1]} with exit code {res.returncode}")
    tmp = LIB + ".tmp"
    res = _run([hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], verbose)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"linking libqift.so failed with exit code {res.returncode}")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
