"""Build libspec_tree.so (gfx950) in-tree with hipcc.

Each HIP source is compiled to an object in ``_build/`` in parallel, then
linked into ``tree_attention_spec_amd/libspec_tree.so``. Run as a script or call
``build()``; it always recompiles.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspec_tree.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "pack.hip", "rope.hip", "attn.hip", "e2etv.hip", "e2etv_head.hip", "gdn.hip", "gdn_chunk.hip"]

# Packed fp32 VALU ops are disabled for device code; hipcc's host pass warns
# that it does not know the feature, which is harmless.
DEVICE_FLAGS = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}", "-I", INCLUDE, "-I", CSRC,
          "-Wall", "-Wno-unused-function", "-Wno-unknown-pragmas"]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (install ROCm or set HIPCC)")


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in r.stdout.splitlines()
                    if "packed-fp32-ops" not in l and "unknown target feature" not in l.lower())
    if r.returncode != 0:
        raise RuntimeError("command failed: %s\n%s" % (" ".join(cmd), r.stdout))
    return out


def build(verbose: bool = False, extra_flags=None) -> str:
    cc = hipcc()
    os.makedirs(BUILD, exist_ok=True)
    flags = COMMON + DEVICE_FLAGS + list(extra_flags or [])

    def compile_one(src):
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        out = _run([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj, out

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES))
    for _, out in results:
        if verbose and out.strip():
            print(out)
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *[o for o, _ in results], "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
