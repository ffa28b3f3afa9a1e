"""Build the HIP library in-tree: top_sampling_vocabs_amd/libqs.so (gfx950).

Usage: python -m top_sampling_vocabs_amd.build  (or build() from Python).
hipcc cross-compiles for gfx950 without a GPU present.
"""

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqs.so")
SOURCES = ["qs_kernels.hip", "qs_api.hip", "qs_spec.hip", "qs_penalty.hip", "qs_toplp.hip"]
ARCH = os.environ.get("QS_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # packed FP32 instructions are kept out of every kernel on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def build(verbose=False):
    """Compile every HIP source into libqs.so next to this file (atomic replace)."""
    srcs = [os.path.join(CSRC, s) for s in SOURCES]
    fd, tmp = tempfile.mkstemp(suffix=".so", dir=PKG)
    os.close(fd)
    cmd = [hipcc()] + HIPCC_FLAGS + srcs + ["-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        os.unlink(tmp)
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}")
    os.chmod(tmp, 0o755)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
