"""Build the gfx950 shared libraries in-tree with hipcc: the layer library
``libmoe_mi355x.so`` and the ablation library ``libmoe_ablation.so``
(token-centric atomic experts, a measurement contrast kept apart).

Usage: python -m mixture_experts_layer_22_amd.build   (or build() from Python)
"""
from __future__ import annotations

import os
import subprocess
import sys
import tempfile

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(HERE, LIB_NAME)
SOURCES = ["api.hip", "router.hip", "dispatch.hip", "gemm.hip", "combine.hip"]
ABL_DIR = os.path.join(HERE, "ablation")
ABL_NAME = "libmoe_ablation.so"
ABL_PATH = os.path.join(HERE, ABL_NAME)
ABL_SOURCES = ["token_centric.hip"]
PRB_DIR = os.path.join(HERE, "probes")
PRB_NAME = "libmoe_probes.so"
PRB_PATH = os.path.join(HERE, PRB_NAME)
PRB_SOURCES = ["probes.hip"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-Wall",
    "-Wno-unused-result",
    # keep the compiler from emitting packed fp32 vector ops
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def _run(cmd):
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout)
        raise RuntimeError(f"hipcc failed ({r.returncode}): {' '.join(cmd)}")
    return r.stdout


def build(verbose: bool = False, jobs: int = 5) -> str:
    """Compile every source for gfx950 and link the layer library (returns
    its path), then the ablation and the ceiling-probe libraries."""
    path = _build_lib(CSRC, SOURCES, LIB_NAME, LIB_PATH, verbose, jobs)
    if os.path.isdir(ABL_DIR):
        _build_lib(ABL_DIR, ABL_SOURCES, ABL_NAME, ABL_PATH, verbose, jobs)
    if os.path.isdir(PRB_DIR):
        _build_lib(PRB_DIR, PRB_SOURCES, PRB_NAME, PRB_PATH, verbose, jobs)
    return path


def _build_lib(src_dir, sources, lib_name, lib_path, verbose, jobs) -> str:
    """Always recompiles (sources are few; each takes seconds).  Objects are
    compiled in parallel into a temporary directory, then linked into
    lib_path atomically."""
    with tempfile.TemporaryDirectory(prefix="moe_build_") as tmp:
        procs = []
        objs = []
        for src in sources:
            obj = os.path.join(tmp, src.replace(".hip", ".o"))
            objs.append(obj)
            cmd = [HIPCC, *FLAGS, "-c", os.path.join(src_dir, src), "-o", obj]
            procs.append((cmd, subprocess.Popen(cmd, stdout=subprocess.PIPE,
                                                stderr=subprocess.STDOUT, text=True)))
            if len([p for _, p in procs if p.poll() is None]) >= jobs:
                procs[-1][1].wait()
        failed = []
        for cmd, p in procs:
            out, _ = p.communicate()
            if p.returncode != 0:
                failed.append((cmd, out))
            elif verbose and out.strip():
                sys.stderr.write(out)
        if failed:
            for cmd, out in failed:
                sys.stderr.write(out)
            raise RuntimeError("hipcc failed: " + "; ".join(" ".join(c[-3:]) for c, _ in failed))
        tmp_lib = os.path.join(tmp, lib_name)
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp_lib])
        os.replace(tmp_lib, lib_path) if os.path.dirname(tmp_lib) == os.path.dirname(lib_path) \
            else _copy(tmp_lib, lib_path)
    return lib_path


def _copy(src, dst):
    tmp = dst + ".tmp"
    with open(src, "rb") as f, open(tmp, "wb") as g:
        g.write(f.read())
    os.replace(tmp, dst)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
