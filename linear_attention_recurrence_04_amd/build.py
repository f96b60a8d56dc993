"""Build libgdn.so (HIP, gfx950) in-tree with hipcc.

Usage: python -m linear_attention_recurrence_04_amd.build
"""
from __future__ import annotations

import glob
import hashlib
import json
import os
import subprocess
import sys
import time

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIBRARY = os.path.join(PKG, "libgdn.so")
BUILD_INFO = os.path.join(PKG, "build_info.json")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed-fp32 VALU ops are kept out of every kernel: -packed-fp32-ops disables
# the target feature for the device pass (the host pass ignores it).
FLAGS = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wno-unused-command-line-argument",
]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def build(verbose: bool = False, out: str = LIBRARY) -> str:
    cmd = [HIPCC] + FLAGS + ["-I", INCLUDE, "-I", CSRC] + sources() + ["-o", out + ".tmp"]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed building libgdn.so")
    os.replace(out + ".tmp", out)
    if out == LIBRARY:
        write_build_info()
    return out


def source_tree_hash() -> str:
    """sha256 (first 16 hex digits) over the library's sources and headers."""
    h = hashlib.sha256()
    for path in sources() + sorted(glob.glob(os.path.join(CSRC, "*.h")) +
                                   glob.glob(os.path.join(CSRC, "*.inc")) +
                                   glob.glob(os.path.join(INCLUDE, "*.h"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _git(*args):
    try:
        r = subprocess.run(["git", "-C", ROOT] + list(args), capture_output=True, text=True,
                           timeout=30)
    except (OSError, subprocess.TimeoutExpired):
        return None
    return r.stdout.strip() if r.returncode == 0 else None


def write_build_info(path: str = BUILD_INFO) -> dict:
    """Record what the library was built from: the git commit (when the tree is
    a git checkout), whether sources differed from it, and the source hash."""
    status = _git("status", "--porcelain", "--", "linear_attention_recurrence_04_amd/csrc",
                  "include")
    info = {"git_sha": _git("rev-parse", "HEAD"),
            "sources_modified_since_commit": (bool(status) if status is not None else None),
            "source_tree_hash": source_tree_hash(),
            "built_utc": time.strftime("%Y-%m-%dT%H:%M:%SZ", time.gmtime()),
            "hipcc_flags": " ".join(FLAGS)}
    with open(path, "w") as f:
        json.dump(info, f, indent=1)
    return info


if __name__ == "__main__":
    print(build(verbose=True))
