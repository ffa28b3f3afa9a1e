"""Build the HIP library in-tree: top_sampling_vocabs_amd/libqs.so (gfx950).

Usage: python -m top_sampling_vocabs_amd.build  (or build() from Python).
hipcc cross-compiles for gfx950 without a GPU present. Each source is compiled
to an object in parallel, then the objects are linked into the library.
"""

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libqs.so")
SOURCES = ["qs_filter_bf16.hip", "qs_filter_f32.hip", "qs_filter_bf16_proc.hip",
           "qs_filter_f32_proc.hip", "qs_filter_bf16_proc1.hip",
           "qs_filter_bf16_sort.hip", "qs_filter_f32_sort.hip", "qs_filter_bf16_topn.hip",
           "qs_filter_f32_topn.hip", "qs_chunk.hip", "qs_api.hip",
           "qs_spec.hip", "qs_penalty.hip", "qs_toplp.hip"]
ARCH = os.environ.get("QS_OFFLOAD_ARCH", "gfx950")

COMPILE_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-fvisibility=hidden",
    "-Wall",
    "-Wno-unused-function",
    # packed FP32 instructions are kept out of every kernel on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
LINK_FLAGS = [f"--offload-arch={ARCH}", "-shared", "-fPIC"]


def hipcc():
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found; the HIP library cannot be built")
    return path


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    return subprocess.run(cmd, capture_output=True, text=True)


def build(verbose=False, jobs=None):
    """Compile every HIP source and link libqs.so next to this file (atomic replace)."""
    cc = hipcc()
    with tempfile.TemporaryDirectory(dir=PKG) as tmpdir:
        objs = [os.path.join(tmpdir, os.path.splitext(s)[0] + ".o") for s in SOURCES]
        cmds = [[cc] + COMPILE_FLAGS + ["-c", os.path.join(CSRC, s), "-o", o]
                for s, o in zip(SOURCES, objs)]
        jobs = jobs or min(len(cmds), os.cpu_count() or 1, 16)
        with ThreadPoolExecutor(max_workers=jobs) as ex:
            results = list(ex.map(lambda c: _run(c, verbose), cmds))
        failed = [(c, r) for c, r in zip(cmds, results) if r.returncode != 0]
        if failed:
            for c, r in failed:
                sys.stderr.write(" ".join(c) + "\n" + r.stdout + r.stderr)
            raise RuntimeError(f"hipcc failed on {len(failed)} source(s)")
        fd, tmp = tempfile.mkstemp(suffix=".so", dir=PKG)
        os.close(fd)
        res = _run([cc] + LINK_FLAGS + objs + ["-o", tmp], verbose)
        if res.returncode != 0:
            os.unlink(tmp)
            sys.stderr.write(res.stdout + res.stderr)
            raise RuntimeError(f"hipcc link failed with exit code {res.returncode}")
    os.chmod(tmp, 0o755)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
