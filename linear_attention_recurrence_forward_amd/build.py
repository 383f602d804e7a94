"""Build libgdn.so (the HIP library behind include/gdn.h) for gfx950.

    python -m linear_attention_recurrence_forward_amd.build

Compiles csrc/gdn_kernels.hip, csrc/gdn_rollback.hip and csrc/gdn_api.cpp into
lib/libgdn.so with hipcc, in-tree. hipcc cross-compiles: no GPU is needed.
"""

from __future__ import annotations

import hashlib
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIBDIR = os.path.join(PKG, "lib")
LIBRARY = os.path.join(LIBDIR, "libgdn.so")
SOURCES = [os.path.join(CSRC, "gdn_kernels.hip"), os.path.join(CSRC, "gdn_rollback.hip"),
           os.path.join(CSRC, "gdn_api.cpp")]
HEADERS = [os.path.join(ROOT, "include", "gdn.h"), os.path.join(CSRC, "gdn_launch.h")]

ARCH = "gfx950"
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
    "-Wall", "-mcode-object-version=5",
    # Keep the compiler from forming packed-FP32 VALU instructions.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Preload the first 13 dwords of kernel arguments into scalar registers
    # at dispatch (the one-token kernel's leading parameters).
    "-mllvm", "-amdgpu-kernarg-preload-count=13",
]


def hipcc() -> str:
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    path = os.path.join(rocm, "bin", "hipcc")
    return path if os.path.exists(path) else "hipcc"


def source_digest() -> str:
    """sha256 over the kernel sources, headers and flags (identifies a build)."""
    h = hashlib.sha256()
    for p in SOURCES + HEADERS:
        with open(p, "rb") as f:
            h.update(f.read())
    h.update(" ".join(FLAGS).encode())
    return h.hexdigest()


def build(verbose: bool = False) -> str:
    os.makedirs(LIBDIR, exist_ok=True)
    tmp = LIBRARY + f".tmp{os.getpid()}"
    cmd = [hipcc(), *FLAGS, f"-I{os.path.join(ROOT, 'include')}", f"-I{CSRC}",
           *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns about the device-only target feature: harmless.
    noise = "'-packed-fp32-ops' is not a recognized feature"
    msgs = [ln for ln in (res.stdout + res.stderr).splitlines() if noise not in ln]
    if res.returncode != 0:
        raise RuntimeError("hipcc failed:\n" + "\n".join(msgs))
    if verbose and msgs:
        print("\n".join(msgs))
    os.replace(tmp, LIBRARY)
    with open(os.path.join(LIBDIR, "libgdn.digest"), "w") as f:
        f.write(source_digest() + "\n")
    return LIBRARY


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
