"""Build libvlp.so in-tree with hipcc for gfx950.

Usage: ``python -m variable_length_packed_pack_amd.build`` (or ``build()``).
Each source compiles to an object under ``_build/`` in parallel, then one
hipcc link produces ``variable_length_packed_pack_amd/libvlp.so``.  Every call
recompiles everything.
"""

from __future__ import annotations

import concurrent.futures
import hashlib
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG_DIR, "csrc")
BUILD_DIR = os.path.join(PKG_DIR, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libvlp.so")

ARCH = "gfx950"
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

COMMON_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-function",
    # Packed fp32 VALU forms are kept out of the generated code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]

SOURCES = [
    "host_meta.cpp",
    "api.cpp",
    "grid_build.hip",
    "attn_first_token.hip",
    "attn_h16.hip",
    "attn_f32.hip",
    "attn_bwd_h16.hip",
    "attn_bwd_f32.hip",
    "ragged_matmul.hip",
    "seq_ids.hip",
    "cu_check.hip",
    "noalloc.hip",
    "calibrate.hip",
]


def source_hash() -> str:
    """First 16 hex digits of a SHA-256 over every file under csrc/ and the
    public header (names and contents, in name order).  The build compiles it
    into the library (vlp_build_info), so a loaded libvlp.so can be matched
    against the sources it claims to come from."""
    h = hashlib.sha256()
    files = sorted(os.path.join("csrc", n) for n in os.listdir(CSRC) if os.path.isfile(os.path.join(CSRC, n)))
    for rel in files + [os.path.join("..", "include", "vlp.h")]:
        with open(os.path.join(PKG_DIR, rel), "rb") as f:
            data = f.read()
        h.update(os.path.basename(rel).encode() + b"\0" + len(data).to_bytes(8, "little") + data)
    return h.hexdigest()[:16]


def _compile(src: str, digest: str) -> tuple[str, str]:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *COMMON_FLAGS, f"-DVLP_SOURCE_HASH=\"{digest}\"", "-c", os.path.join(CSRC, src), "-o", obj]
    if src.endswith(".hip"):
        cmd[1:1] = ["-x", "hip"]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    return obj, res.stderr


def build(verbose: bool = False, jobs: int | None = None) -> str:
    """Compile every source and link libvlp.so; returns the library path."""
    if not os.path.exists(HIPCC):
        raise RuntimeError(f"hipcc not found at {HIPCC}")
    os.makedirs(BUILD_DIR, exist_ok=True)
    jobs = jobs or min(len(SOURCES), max(1, (os.cpu_count() or 4)))
    digest = source_hash()
    with concurrent.futures.ThreadPoolExecutor(max_workers=jobs) as ex:
        results = list(ex.map(lambda src: _compile(src, digest), SOURCES))
    objs = [r[0] for r in results]
    if verbose:
        for src, (_, err) in zip(SOURCES, results):
            if err.strip():
                print(f"--- {src}\n{err}", file=sys.stderr)
    tmp = LIB_PATH + ".tmp"
    # -z defs: an unresolved symbol (such as a kernel stub the host pass did
    # not emit) fails the link instead of the first dlopen.
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-Wl,-z,defs", *objs, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{res.stdout}\n{res.stderr}")
    shutil.move(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
