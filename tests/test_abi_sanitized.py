"""The C ABI layer under AddressSanitizer and UndefinedBehaviorSanitizer (host code).

spatially_sharded_conv_amd/build_sanitized.py builds libvaep_san.so with both sanitizers on
the host pass; this test runs tests/test_abi_cpu.py against it in a child process that
preloads clang's ASan runtime (which also carries the UBSan handlers).  Any heap or stack
overflow, use after free or undefined behaviour in argument validation, configuration,
sizing and error reporting aborts the child.  CPU only.
"""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# what the child checks before running the ABI tests: the sanitized library and the ASan
# runtime are the ones in the process
PROBE = r"""
import ctypes, sys
from spatially_sharded_conv_amd import _lib as L
L.load()
maps = open("/proc/self/maps").read()
assert "libvaep_san.so" in maps and "libclang_rt.asan" in maps, "sanitized build not loaded"
ctypes.CDLL(None).__asan_region_is_poisoned   # the ASan runtime is live
print("sanitized library loaded:", L.LIB_PATH)
"""


def _toolchain():
    if not (os.environ.get("HIPCC") or os.path.exists("/opt/rocm/bin/hipcc") or shutil.which("hipcc")):
        return None
    from spatially_sharded_conv_amd import build_sanitized as bs
    return bs


def test_abi_checks_under_address_and_ub_sanitizers():
    bs = _toolchain()
    if bs is None:
        pytest.skip("hipcc not available")
    rt = bs.asan_runtime()
    if rt is None:
        pytest.skip("clang ASan runtime not found next to hipcc")
    lib = bs.build(verbose=False)
    env = dict(os.environ)
    env.update(LD_PRELOAD=rt, VAEP_LIB=lib, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    probe = subprocess.run([sys.executable, "-c", PROBE], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
    assert probe.returncode == 0, probe.stdout + probe.stderr
    r = subprocess.run([sys.executable, "-m", "pytest", "tests/test_abi_cpu.py", "-q", "-p", "no:cacheprovider"],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out and "runtime error:" not in out, out[-4000:]
    assert r.returncode == 0 and " passed" in out, out[-4000:]
