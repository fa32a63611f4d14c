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
# ceiling probes for the roofline figures: a library of its own, loaded only by the
# benchmark's ceiling mode
PROBE_SOURCE = "probe.hip"
PROBE_LIB = os.path.join(PKG, "libspec_probe.so")
ARCH = "gfx950"

SOURCES = ["abi.hip", "pack.hip", "rope.hip", "attn.hip", "qsa.hip", "e2etv.hip", "e2etv_head.hip", "gdn.hip",
           "gdn_chunk.hip"]

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

    with ThreadPoolExecutor(min(len(SOURCES) + 1, os.cpu_count() or 1)) as ex:
        results = list(ex.map(compile_one, SOURCES + [PROBE_SOURCE]))
    for _, out in results:
        # compiler warnings are always shown (the packed-fp32 host note is filtered in _run)
        lines = [l for l in out.splitlines() if verbose or "warning" in l or "error" in l]
        if lines:
            print("\n".join(lines))
    objs = [o for o, _ in results]
    probe_obj = objs.pop()
    tmp = LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", probe_obj, "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


# Host-side sanitizers for the CPU tests: AddressSanitizer and UBSan apply to the
# host code only (argument checks, size queries, the pack plan); device code is
# built as usual.
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-fno-sanitize-recover=undefined"]
HOST_SAN_LIB = os.path.join(BUILD, "hostsan", "libspec_tree_hostsan.so")


def asan_runtime() -> str:
    """The clang AddressSanitizer runtime that a host-sanitized library needs preloaded."""
    import glob
    cands = sorted(glob.glob("/opt/rocm/lib/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not cands:
        raise RuntimeError("clang AddressSanitizer runtime not found under /opt/rocm/lib/llvm")
    return cands[-1]


def build_host_sanitized() -> str:
    """libspec_tree with host code under ASan + UBSan, in _build/hostsan/ (not the product)."""
    cc = hipcc()
    out_dir = os.path.dirname(HOST_SAN_LIB)
    os.makedirs(out_dir, exist_ok=True)
    flags = ["-O1", "-g"] + COMMON[1:] + DEVICE_FLAGS + HOST_SAN

    def compile_one(src):
        obj = os.path.join(out_dir, src.replace(".hip", ".o"))
        _run([cc, *flags, "-c", os.path.join(CSRC, src), "-o", obj])
        return obj

    with ThreadPoolExecutor(min(len(SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = HOST_SAN_LIB + ".tmp"
    _run([cc, "-shared", "-fPIC", f"--offload-arch={ARCH}", *HOST_SAN, *objs, "-o", tmp])
    os.replace(tmp, HOST_SAN_LIB)
    return HOST_SAN_LIB


if __name__ == "__main__":
    if "--host-sanitized" in sys.argv:
        print(build_host_sanitized())
    else:
        print(build(verbose="-v" in sys.argv))
