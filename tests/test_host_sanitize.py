"""Host code under AddressSanitizer and UBSan (CPU only).

The library is rebuilt with `-Xarch_host -fsanitize=address,undefined` (device code
as usual) into _build/hostsan/, and the C-ABI CPU tests — argument checks, size
queries and the host pack plan of every workload — run against it in a child
process with the clang ASan runtime preloaded. Any report fails the test."""
import importlib.util
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _build_module():
    spec = importlib.util.spec_from_file_location(
        "spec_build", os.path.join(ROOT, "tree_attention_spec_amd", "build.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


@pytest.mark.skipif(not (os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")),
                    reason="hipcc not available")
def test_abi_cpu_tests_under_host_asan_ubsan():
    b = _build_module()
    try:
        rt = b.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = b.build_host_sanitized()
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, SPEC_TREE_LIBRARY=lib,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1:abort_on_error=0",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_abi_cpu.py")],
                       cwd=ROOT, env=env, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True,
                       timeout=600)
    out = r.stdout
    print(out[-3000:])
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert r.returncode == 0
    assert " passed" in out
