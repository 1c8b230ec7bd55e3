"""Build libpa_decode.so (the gfx950 HIP library) in-tree with hipcc.

Every translation unit under csrc/ is compiled for gfx950 only, in parallel,
then linked into ``_lib/libpa_decode.so`` next to this file. Packed fp32 VALU
instructions are disabled for all device code; no fast-math or denormal
flushing is requested, so divisions and square roots stay correctly rounded.
"""
from __future__ import annotations

import concurrent.futures
import glob
import hashlib
import json
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD_DIR = os.path.join(HERE, "_build")
LIB_DIR = os.path.join(HERE, "_lib")
LIB_PATH = os.path.join(LIB_DIR, "libpa_decode.so")
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
COMMON = [
    "-std=c++17", "-O3", "-fPIC", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # MFMA accumulators in ordinary VGPRs: the decode rescales them with vector
    # ALU ops, which would otherwise copy them out of and back into AGPRs
    "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall", "-Wno-unused-parameter", "-Wno-unknown-pragmas",
]


def _sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "pa_api.cpp")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [HIPCC, *COMMON, "-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    return obj


def build(jobs: int = 0) -> str:
    """Compile all sources and link the shared library; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    os.makedirs(LIB_DIR, exist_ok=True)
    srcs = _sources()
    jobs = jobs or min(len(srcs), max(1, min(os.cpu_count() or 4, 16)))
    with concurrent.futures.ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, srcs))
    tmp = LIB_PATH + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", f"--offload-arch={ARCH}", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
    os.replace(tmp, LIB_PATH)
    _write_build_info(srcs)
    return LIB_PATH


def _write_build_info(srcs) -> None:
    """Record what the library was built from (the commit, when this is a git
    checkout, and a digest of the sources), next to the library: runs on a
    copy of the tree without its history can still name their build."""
    h = hashlib.sha256()
    for src in srcs + [os.path.join(HERE, "..", "include", "pa_decode.h")]:
        h.update(open(src, "rb").read())
    head = None
    try:
        r = subprocess.run(["git", "-C", HERE, "rev-parse", "HEAD"], capture_output=True, text=True, timeout=10)
        if r.returncode == 0:
            head = r.stdout.strip()
            d = subprocess.run(["git", "-C", HERE, "status", "--porcelain", "--untracked-files=no"],
                               capture_output=True, text=True, timeout=10)
            if d.returncode == 0 and d.stdout.strip():
                head += "+uncommitted"
    except (OSError, subprocess.SubprocessError):
        pass
    with open(os.path.join(LIB_DIR, "build_info.json"), "w") as f:
        json.dump({"git_head": head, "source_digest": h.hexdigest()[:16]}, f)


if __name__ == "__main__":
    print(build())
    sys.exit(0)
