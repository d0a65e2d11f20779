"""Host-sanitized build of the library for CPU-side checks of the C ABI layer.

Compiles the same sources as build.py into _build_san/ and links libvaep_san.so, with
AddressSanitizer and UndefinedBehaviorSanitizer on the host pass only (device code is
built as usual).  The sanitizer runtime is not linked in: a process that loads this
library preloads clang's ASan runtime (asan_runtime() below), which also carries the
UBSan handlers.  Used by tests/test_abi_sanitized.py; never by the product path.

Usage: python -m spatially_sharded_conv_amd.build_sanitized
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

from spatially_sharded_conv_amd.build import CSRC, FILE_FLAGS, FLAGS, HERE, SOURCES, hipcc

OUT = os.path.join(HERE, "libvaep_san.so")
OBJ = os.path.join(HERE, "_build_san")
# every sanitizer flag goes to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all", "-Xarch_host", "-fno-omit-frame-pointer",
            "-Xarch_host", "-g"]


def asan_runtime() -> str | None:
    """Path of clang's shared ASan runtime next to hipcc, or None."""
    root = os.path.dirname(os.path.dirname(os.path.realpath(hipcc())))
    for cand in sorted(glob.glob(os.path.join(root, "llvm", "lib", "clang", "*", "lib", "linux",
                                              "libclang_rt.asan-x86_64.so"))):
        return cand
    return None


def _compile(src: str) -> str:
    obj = os.path.join(OBJ, os.path.splitext(src)[0] + ".o")
    path = os.path.join(CSRC, src)
    if os.path.exists(obj) and os.path.getmtime(obj) >= max(
            os.path.getmtime(p) for p in glob.glob(os.path.join(CSRC, "*")) + [path]):
        return obj
    cmd = [hipcc()] + FLAGS + FILE_FLAGS.get(src, []) + HOST_SAN + ["-c", path, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile of {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(len(SOURCES), os.cpu_count() or 4)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    tmp = OUT + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, OUT)
    if verbose:
        print(f"built {OUT}")
    return OUT


if __name__ == "__main__":
    build()
    sys.exit(0)
