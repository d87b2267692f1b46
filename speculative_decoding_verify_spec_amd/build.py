"""Build libspec_verify.so (HIP, gfx950) in the package directory.

Every .hip file under csrc/ is compiled to an object in _build/ (in parallel)
and linked into one shared library exporting the C ABI of
include/spec_verify.h.  Run `python -m speculative_decoding_verify_spec_amd.build`.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libspec_verify.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
    # no packed fp32 instructions in device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-result", "-I" + os.path.join(ROOT, "include"),
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


# Host-side AddressSanitizer variant (device code unchanged): every host
# function of the runtime instrumented, for the CPU checks of the C ABI.  The
# sanitizer flags apply to the host compilation only.
ASAN_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]


def build_host_asan(out_dir: str) -> str:
    """Build <out_dir>/libspec_verify.so with host ASan; skipped when the
    sources are unchanged since the last such build.  Returns the path."""
    import hashlib

    os.makedirs(out_dir, exist_ok=True)
    srcs = sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.h")) +
                  glob.glob(os.path.join(ROOT, "include", "*.h")))
    h = hashlib.sha256()
    for f in srcs:
        with open(f, "rb") as fh:
            h.update(os.path.basename(f).encode() + fh.read())
    key = h.hexdigest()
    lib = os.path.join(out_dir, "libspec_verify.so")
    stamp = os.path.join(out_dir, "sources.sha256")
    if os.path.exists(lib) and os.path.exists(stamp) and open(stamp).read().strip() == key:
        return lib

    def one(src):
        obj = os.path.join(out_dir, os.path.basename(src) + ".o")
        cmd = [HIPCC, *FLAGS, *ASAN_HOST, "-g", "-c", src, "-o", obj]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
        return obj

    hips = sorted(glob.glob(os.path.join(CSRC, "*.hip")))
    with cf.ThreadPoolExecutor(max_workers=min(8, len(hips))) as ex:
        objs = list(ex.map(one, hips))
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", *objs, "-o", lib]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    with open(stamp, "w") as fh:
        fh.write(key + "\n")
    return lib


if __name__ == "__main__":
    build()
    sys.exit(0)
