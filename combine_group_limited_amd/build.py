"""Build libep.so (the HIP library) in-tree with hipcc for gfx950.

Usage: python -m combine_group_limited_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import hashlib
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(PKG, "_build")
LIB_PATH = os.path.join(PKG, "libep.so")
# HBM bandwidth probes used by the benchmark's ceiling probe (not part of
# the library's ABI)
PROBE_LIB_PATH = os.path.join(PKG, "libhbmprobe.so")
PROBE_SOURCES = ["probe.hip"]
# device self-checks run by the test suite (not part of the library's ABI)
CHECK_LIB_PATH = os.path.join(PKG, "libepcheck.so")
CHECK_SOURCES = ["selfcheck.hip"]
# content hash of the sources and flags the library was built from, written
# next to it by build(); the loader compares it with the current sources
HASH_PATH = LIB_PATH + ".sources"

SOURCES = ["api.hip", "gate.hip", "layout.hip", "dispatch.hip", "combine.hip", "ll.hip"]
HEADERS = ["device.h", "launch.h", "rows.h"]

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")

# -ffp-contract=off: fp32 expressions are evaluated as written (explicit
# fmaf only), which the bit-exact routing and quantisation rely on.
# -packed-fp32-ops off: no packed fp32 arithmetic in device code.
HIPFLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",
    "-fno-fast-math",
    "-fvisibility=hidden",
    "-mcode-object-version=5",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", INCLUDE,
    "-I", CSRC,
]


def _inputs():
    return [os.path.join(CSRC, f) for f in SOURCES + PROBE_SOURCES + CHECK_SOURCES + HEADERS] + \
        [os.path.join(INCLUDE, "ep.h")]


def source_hash(inputs=None) -> str:
    """SHA-256 over the compiler flags (include directories by name only, so
    that a copy of the tree at another path matches) and the name and bytes
    of every input."""
    flags = [os.path.basename(f) if os.path.isabs(f) else f for f in HIPFLAGS]
    h = hashlib.sha256("\0".join(flags).encode())
    for p in (inputs if inputs is not None else _inputs()):
        h.update(os.path.basename(p).encode() + b"\0")
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def built_hash():
    """The source hash recorded when libep.so was built, or None."""
    try:
        with open(HASH_PATH) as f:
            return f.read().strip()
    except OSError:
        return None


def is_stale() -> bool:
    """True when libep.so is missing or was built from other sources or
    flags than the current ones (compared by content, not by time stamps,
    which a copied tree need not keep)."""
    return (not os.path.exists(LIB_PATH) or not os.path.exists(PROBE_LIB_PATH)
            or not os.path.exists(CHECK_LIB_PATH) or built_hash() != source_hash())


def hipcc_available() -> bool:
    return os.path.exists(HIPCC) or shutil.which(HIPCC) is not None


def _compile(src: str) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(os.path.basename(src))[0] + ".o")
    cmd = [HIPCC, *HIPFLAGS, "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed for %s:\n%s\n%s" % (src, " ".join(cmd), r.stderr))
    # hipcc's host pass does not know the packed-fp32 target feature; that
    # warning is expected, anything else is shown
    for line in r.stderr.splitlines():
        if "packed-fp32-ops" not in line and line.strip():
            print(line, file=sys.stderr)
    return obj


def build(verbose: bool = False) -> str:
    """Compile every HIP source and link libep.so (and the benchmark's
    libhbmprobe.so and the tests' libepcheck.so) next to this file."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    digest = source_hash()
    srcs = [os.path.join(CSRC, f) for f in SOURCES + PROBE_SOURCES + CHECK_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(_compile, srcs))
    n, p = len(SOURCES), len(PROBE_SOURCES)
    for path, part in ((LIB_PATH, objs[:n]), (PROBE_LIB_PATH, objs[n:n + p]), (CHECK_LIB_PATH, objs[n + p:])):
        tmp = path + ".tmp%d" % os.getpid()
        cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *part]
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n%s\n%s" % (" ".join(cmd), r.stderr))
        os.replace(tmp, path)
    tmp = HASH_PATH + ".tmp%d" % os.getpid()
    with open(tmp, "w") as f:
        f.write(digest + "\n")
    os.replace(tmp, HASH_PATH)
    if verbose:
        print("built", LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    build(verbose=True)
