"""Compile the HIP library (libpkv.so) for gfx950, in-tree.

Every .hip/.cpp file under csrc/ is compiled with hipcc to an object in
_build/, in parallel, and linked into paged_attention_kv_store_amd/libpkv.so.
Packed-fp32 instructions are disabled for the device code.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpkv.so")
ARCH = os.environ.get("PKV_OFFLOAD_ARCH", "gfx950")

HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
    "-Wall", "-Wno-unused-function",
]


def sources():
    return sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC)
                  if f.endswith((".hip", ".cpp")))


def _scratch_users(remarks):
    """Kernels whose resource-usage remarks report scratch (private) memory."""
    users, name = [], None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and int(m.group(1)) > 0 and name:
            users.append((name, int(m.group(1))))
    return users


def _compile(src, verbose):
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC, *FLAGS, "-Rpass-analysis=kernel-resource-usage", "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # the host pass does not know the packed-fp32 feature; that warning is noise
    noise = "is not a recognized feature for this target"
    lines = [l for l in res.stderr.splitlines() if noise not in l]
    err = "\n".join(l for l in lines if "kernel-resource-usage" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    # A kernel that spills to or keeps arrays in scratch memory runs far
    # slower than intended; treat it as a build error.
    users = _scratch_users("\n".join(lines))
    if users:
        raise RuntimeError(f"kernels in {src} use scratch memory: {users}")
    return obj


def build(verbose: bool = False, jobs: int | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = sources()
    jobs = jobs or min(len(srcs), int(os.environ.get("MAX_JOBS", os.cpu_count() or 4)), 16)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), srcs))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{res.stderr}")
    os.replace(tmp, LIB)
    return LIB


PROBE_SRC = os.path.join(PKG, "probe", "hbm_read.hip")
PROBE_LIB = os.path.join(PKG, "libpkv_probe.so")


def build_probe(verbose: bool = False) -> str:
    """The benchmark's streaming-read kernel (a measurement aid, kept out of
    libpkv.so): libpkv_probe.so."""
    tmp = PROBE_LIB + ".tmp"
    cmd = [HIPCC, *FLAGS, "-shared", PROBE_SRC, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed on {PROBE_SRC}:\n{res.stderr}")
    os.replace(tmp, PROBE_LIB)
    return PROBE_LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    print(build_probe(verbose="-v" in sys.argv))
