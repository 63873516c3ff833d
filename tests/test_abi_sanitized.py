"""The C ABI's host-side checks under AddressSanitizer and
UndefinedBehaviorSanitizer (CPU only).

abi.cpp (argument validation, overlap checks, workspace layout, launch
sequencing) is rebuilt with host ASan + UBSan (linear_compressed_attention_amd/
build_sanitized.py) and tests/test_abi_host.py runs against that build in a
child process with the ASan runtime preloaded: every call path those tests
reach (bad shapes, null / misaligned / overlapping pointers, short
workspaces, layouts, the missing-device report) runs instrumented, and any
memory error or undefined behaviour ends the child with a report.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

_CHILD = r"""
import importlib.util, os, sys
tmp, root = sys.argv[1], sys.argv[2]
sys.path.insert(0, root)
pkg = os.path.join(tmp, "linear_compressed_attention_amd")
spec = importlib.util.spec_from_file_location("linear_compressed_attention_amd", os.path.join(pkg, "__init__.py"),
                                              submodule_search_locations=[pkg])
mod = importlib.util.module_from_spec(spec)
sys.modules["linear_compressed_attention_amd"] = mod
spec.loader.exec_module(mod)
assert mod.lib_path().startswith(tmp), mod.lib_path()
import pytest
sys.exit(pytest.main(["-q", "-x", "-s", "-p", "no:cacheprovider", "-m", "not gpu",
                      os.path.join(root, "tests", "test_abi_host.py")]))
"""


def test_abi_host_checks_under_host_sanitizers(tmp_path):
    if not os.path.exists("/opt/rocm/bin/hipcc"):
        pytest.skip("needs hipcc")
    sys.path.insert(0, os.path.join(ROOT, "linear_compressed_attention_amd"))
    try:
        import build_sanitized as BS
    finally:
        sys.path.pop(0)
    out = tmp_path / "san"
    lib = BS.build_sanitized(str(out))
    pkg = tmp_path / "linear_compressed_attention_amd"
    pkg.mkdir()
    shutil.copy(os.path.join(ROOT, "linear_compressed_attention_amd", "__init__.py"), pkg / "__init__.py")
    shutil.copy(lib, pkg / "libedit_attn.so")
    shutil.copytree(os.path.join(ROOT, "include"), tmp_path / "include")
    env = dict(os.environ)
    env["LD_PRELOAD"] = BS.asan_runtime()
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:abort_on_error=0:exitcode=86"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1:exitcode=87"
    r = subprocess.run([sys.executable, "-c", _CHILD, str(tmp_path), ROOT], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    tail = (r.stdout + r.stderr)[-4000:]
    assert "AddressSanitizer" not in tail and "runtime error" not in tail, tail
    assert r.returncode == 0, tail
    assert " passed" in r.stdout, tail
