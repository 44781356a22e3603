"""The host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libmimo_attn_hostsan.so is the library's host code alone (argument validation, split planning,
head grouping, the error paths and messages; no device code), built with both sanitizers. The
C-ABI tests (tests/test_abi_cpu.py) run against it in a child process whose sanitizer runtime is
preloaded ahead of whatever the environment already preloads; any report fails this test. No GPU
is needed: every call in those tests is rejected by validation before a launch.
"""

import glob
import os
import subprocess
import sys

import pytest

from sliding_window_sink_seeded_amd import build

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = """
import sys
sys.path.insert(0, {tests!r})
import sliding_window_sink_seeded_amd as mimo
mimo.LIB_PATH = {lib!r}
import pytest
rc = pytest.main(["-q", "-p", "no:cacheprovider", {abi!r}])
assert mimo.library()._name == {lib!r}
sys.exit(int(rc))
"""


def test_abi_tests_pass_under_host_sanitizers():
    if not os.path.exists(build.LIB_HOSTSAN):
        pytest.skip("libmimo_attn_hostsan.so not built")
    rt = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not rt:
        pytest.skip("no AddressSanitizer runtime in this ROCm installation")
    env = dict(os.environ)
    env["LD_PRELOAD"] = " ".join(x for x in (rt[-1], os.environ.get("LD_PRELOAD", "")) if x)
    env["ASAN_OPTIONS"] = "detect_leaks=0:halt_on_error=1:verify_asan_link_order=0"
    env["UBSAN_OPTIONS"] = "halt_on_error=1:print_stacktrace=1"
    code = CHILD.format(tests=os.path.join(ROOT, "tests"), lib=build.LIB_HOSTSAN,
                        abi=os.path.join(ROOT, "tests", "test_abi_cpu.py"))
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True,
                       timeout=600, cwd=ROOT)
    out = r.stdout + r.stderr
    assert r.returncode == 0, out[-4000:]
    for marker in ("runtime error:", "AddressSanitizer", "UndefinedBehaviorSanitizer"):
        assert marker not in out, out[-4000:]
