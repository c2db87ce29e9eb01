"""Build of the library with AddressSanitizer and UndefinedBehaviorSanitizer on its host code,
for the C-ABI argument checks run without a GPU (the device code is compiled as
usual; the host checks reject their arguments before any kernel launch).  The build
is cached under <repo>/_build/host_sanitized and redone when a source or flag changes.
"""
from __future__ import annotations

import glob
import hashlib
import os
import subprocess
from concurrent.futures import ThreadPoolExecutor

from sequence_compressed_kv_amd import build as B

OUT = os.path.join(B.BUILD, "host_sanitized")
LIB = os.path.join(OUT, "libsckv_host_sanitized.so")
CLANG = "/opt/rocm/llvm/bin/clang++"
# every sanitizer flag applies to the host pass only
SAN = ["-Xarch_host", "-fsanitize=address",
       "-Xarch_host", "-fsanitize=undefined",
       "-Xarch_host", "-fno-sanitize-recover=undefined",
       "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
LINK = [CLANG, "-shared", "-fPIC", "-fsanitize=address,undefined", "-shared-libsan"]


def runtime() -> str:
    """The shared AddressSanitizer runtime (UBSan's handlers included) to preload."""
    found = sorted(glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not found:
        raise FileNotFoundError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return found[-1]


def _key() -> str:
    h = hashlib.sha256()
    for f in sorted(os.listdir(B.CSRC)) + ["sckv.h"]:
        path = os.path.join(B.INCLUDE if f == "sckv.h" else B.CSRC, f)
        with open(path, "rb") as fh:
            h.update(f.encode() + fh.read())
    h.update(" ".join(B.FLAGS + SAN + LINK).encode())
    return h.hexdigest()


def _compile(src: str) -> str:
    obj = os.path.join(OUT, os.path.splitext(src)[0] + ".o")
    cmd = [B.HIPCC, *B.FLAGS, *SAN, "-x", "hip", "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host build of {src} failed:\n{r.stderr}")
    return obj


def build() -> str:
    key = _key()
    stamp = os.path.join(OUT, "key")
    if os.path.exists(LIB) and os.path.exists(stamp) and open(stamp).read() == key:
        return LIB
    os.makedirs(OUT, exist_ok=True)
    with ThreadPoolExecutor(min(len(B.SOURCES), os.cpu_count() or 1)) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    r = subprocess.run([*LINK, *objs, "-L/opt/rocm/lib", "-lamdhip64", "-Wl,-rpath,/opt/rocm/lib", "-o", LIB],
                       capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"sanitized host link failed:\n{r.stderr}")
    with open(stamp, "w") as f:
        f.write(key)
    return LIB
