"""Compiles the HIP sources under ``csrc/`` into ``libconvmi.so`` for gfx950.

Objects go to ``_build/`` beside this file; the shared library is written
in-tree next to this file so that it travels with the source tree.
"""
from __future__ import annotations

import concurrent.futures
import glob
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libconvmi.so")
# Host code under AddressSanitizer and UndefinedBehaviorSanitizer (the device
# code is built as usual); loaded instead of LIB when CONVMI_SANITIZED=1.
OBJ_SAN = os.path.join(PKG, "_build_san")
LIB_SAN = os.path.join(PKG, "libconvmi_san.so")
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
             "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
CFLAGS = [
    "-O3",
    "-std=c++17",
    f"--offload-arch={ARCH}",
    "-fPIC",
    # No packed-fp32 instructions anywhere in the device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
    "-Wall",
]


def _compile(src: str, sanitize: bool = False) -> str:
    obj = os.path.join(OBJ_SAN if sanitize else OBJ, os.path.basename(src) + ".o")
    flags = [f for f in CFLAGS if f != "-O3"] + ["-O1", "-g"] + SAN_FLAGS if sanitize else CFLAGS
    cmd = [HIPCC, *flags, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(jobs: int = 8, sanitize: bool = False) -> str:
    """Compile every ``csrc/*.hip`` and link ``libconvmi.so`` (with
    ``sanitize``: ``libconvmi_san.so``, host code under ASan and UBSan);
    returns its path."""
    os.makedirs(OBJ_SAN if sanitize else OBJ, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda f: _compile(f, sanitize), srcs))
    lib = LIB_SAN if sanitize else LIB
    tmp = lib + ".tmp"
    link = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    if sanitize:
        link[1:1] = SAN_FLAGS[:4] + ["-shared-libasan"]
    r = subprocess.run(link, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)
    return lib


if __name__ == "__main__":
    print(build())
